"""Summaries of rocprofv3 output for the profiles/ folder.

    python profsum.py trace STATS_CSV --title T --command C
        kernel-trace statistics (``rocprofv3 --kernel-trace --stats --output-format csv``)
        as a markdown table.

    python profsum.py counters --fetch CSV --write CSV \
            --workload NAME --mode decode|prefill --calib-bytes N --fetch-command C --write-command C
        HBM traffic per launch of each kernel of the path, from two ``rocprofv3 --pmc`` runs
        of ``bench.py --pmc-pass`` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Both
        counters are scaled by what they read for the calibration kernel at the end of the
        pass, a plain elementwise kernel (torch.neg on bf16) that reads N bytes and writes N
        bytes: traffic = FETCH_SIZE * 1024 * N / FETCH_calib + WRITE_SIZE * 1024 * N / WRITE_calib.
        The output carries the digest of the kernel sources it was taken on; bench.py reports
        the traffic only while the sources still have that digest.

    python profsum.py mfma CSV --workload NAME --mode decode|prefill \
            --command C [--xcds 8] [--simds 1024]
        MFMA use per kernel of the path from one ``rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
        GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16`` run: MFMA busy cycles per SIMD, the
        fraction of the dispatch's duration they fill at the nominal clock (= the fraction of
        the nominal bf16 peak), and the bf16 MFMA flops the hardware counted (MOPS x 512).
"""
import argparse
import csv
import hashlib
import os
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))

# kernel function name -> name of the step in lora_linear_profiled / bench.py
_STEP_OF_KERNEL = [
    ("decode_gemm_kernel", "decode_gemm_lora"),
    ("decode_gemm_fp8_kernel", "decode_gemm_fp8"),
    ("decode_gemm_fp8_lora_kernel", "decode_gemm_fp8_lora"),
    ("reduce_lora_kernel", "decode_reduce_lora"),
    ("reduce_seg_kernel", "decode_reduce_lora"),
    ("build_segments_kernel", "build_segments"),
    ("build_segments_small_kernel", "build_segments"),
    ("shrink_finalize_kernel", "shrink_finalize"),
    ("shrink_mfma_kernel", "shrink"),
    ("splitk_reduce_kernel", "splitk_reduce"),
    ("sk_reduce_lora_kernel", "decode_reduce_lora"),
    ("expand_kernel", "expand"),
    ("gemm_big_kernel", "gemm"),
    ("gemm_kernel", "gemm"),
    ("gemm_sk_kernel", "gemm"),
    ("moe_gemm_kernel", "moe_gemm"),
    ("moe_reduce_kernel", "moe_reduce"),
]
_CALIB = "neg_kernel"


def kernel_sources_digest() -> str:
    """sha256 (16 hex digits) over the names and bytes of the library's csrc/*.hip, *.h, *.cpp."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rank_adapter_gemm_sgmv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def short_name(n: str) -> str:
    n = n.replace("(anonymous namespace)::", "").replace("void ", "")
    n = re.sub(r"\((?!anon).*$", "", n)
    return n.replace("lora::", "")[:90]


def step_of(kernel_name: str, mode: str, separate_shrink: bool = False):
    """Step of a kernel; the decode GEMM is "decode_gemm" where a separate shrink kernel
    ran beside it (batches of 129-256 rows), else the fused "decode_gemm_lora"."""
    base = short_name(kernel_name)
    fn = base.split("<")[0]
    for k, step in _STEP_OF_KERNEL:
        if fn == k:
            if step == "gemm":
                return "gemm_prefill_lora" if mode == "prefill" else "gemm_decode"
            if step == "decode_gemm_lora" and separate_shrink:
                return "decode_gemm"
            return step
    return None


def dispatch_medians(trace_csv: str) -> dict:
    """Median duration (ns) per kernel name over the dispatches of a kernel-trace CSV."""
    by = {}
    for r in csv.DictReader(open(trace_csv)):
        by.setdefault(r["Kernel_Name"], []).append(
            float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    out = {}
    for k, v in by.items():
        v = sorted(v)
        n = len(v)
        out[k] = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return out


def trace_table(stats_csv: str, title: str, command: str) -> str:
    """The stats CSV as a table; with the kernel-trace CSV beside it (same prefix), a median
    column too (the average also counts the cold calls the benchmark makes on purpose)."""
    rows = list(csv.DictReader(open(stats_csv)))
    trace = stats_csv.replace("_kernel_stats.csv", "_kernel_trace.csv")
    med = dispatch_medians(trace) if trace != stats_csv and os.path.exists(trace) else {}
    out = [f"# {title}", "", "Command (from the repository root on the GPU host):", "", "```",
           command, "```", "", "| kernel | calls | avg us | median us | min us | max us | % of GPU time |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        m = med.get(r["Name"])
        ms = f"{m / 1e3:.2f}" if m is not None else "-"
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{ms} | {float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def per_dispatch(counter_csv: str, counter: str):
    """[(kernel name, value in KiB)] per dispatch, in dispatch order."""
    acc = {}
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        name, v = acc.get(key, (r["Kernel_Name"], 0.0))
        acc[key] = (name, v + float(r["Counter_Value"]))
    return [acc[k] for k in sorted(acc)]


def counters_table(fetch_csv, write_csv, workload, mode, calib_bytes, fetch_cmd, write_cmd) -> str:
    f = per_dispatch(fetch_csv, "FETCH_SIZE")
    w = per_dispatch(write_csv, "WRITE_SIZE")

    def calib(rows, what):
        vals = [v for n, v in rows if _CALIB in n]
        if not vals:
            raise SystemExit(f"no calibration kernel ({_CALIB}) in the {what} run")
        return sum(vals) / len(vals)

    cf, cw = calib(f, "FETCH_SIZE"), calib(w, "WRITE_SIZE")
    ff = cf * 1024 / calib_bytes  # counter bytes per real byte read
    fw = cw * 1024 / calib_bytes

    def by_step(rows):
        d = {}
        sep = any(step_of(n, mode) == "shrink" for n, _ in rows)
        for n, v in rows:
            s = step_of(n, mode, sep)
            if s is not None:
                d.setdefault(s, []).append(v)
        return d

    fs, ws = by_step(f), by_step(w)
    out = [f"# HBM traffic per launch: {workload} ({mode})", "",
           f"sources_digest: {kernel_sources_digest()}", "",
           "Commands (from the repository root on the GPU host), one counter per run:", "", "```",
           fetch_cmd, write_cmd, "```", "",
           f"Calibration: torch.neg over {calib_bytes} bytes of bf16 (reads and writes {calib_bytes} "
           f"bytes): FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB per dispatch, so the counters "
           f"read {ff:.3f}x (fetch) and {fw:.3f}x (write) the bytes moved.", "",
           "| step | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | traffic MB per launch (calibrated) |",
           "|---|---|---|---|---|"]
    lines = []
    for step in sorted(set(fs) | set(ws)):
        fv = fs.get(step, [0.0])
        wv = ws.get(step, [0.0])
        fk, wk = sum(fv) / len(fv), sum(wv) / len(wv)
        traffic = fk * 1024 / ff + wk * 1024 / fw
        out.append(f"| {step} | {len(fv)} | {fk:.0f} | {wk:.0f} | {traffic / 1e6:.2f} |")
        lines.append(f"traffic {step} {traffic:.0f}")
    out += ["", "Per-launch calibrated bytes, as read by bench.py:", "", "```", *lines, "```", ""]
    return "\n".join(out)


def per_dispatch_full(counter_csv: str):
    """{dispatch: {"name", "ns", counter: summed value}} from a counter-collection CSV."""
    acc = {}
    for r in csv.DictReader(open(counter_csv)):
        key = int(r["Dispatch_Id"])
        d = acc.setdefault(key, {"name": r["Kernel_Name"],
                                 "ns": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return acc


def mfma_table(csv_path, workload, mode, command, xcds=8, simds=1024, ghz=2.4) -> str:
    rows = per_dispatch_full(csv_path)
    sep = any(step_of(d["name"], mode) == "shrink" for d in rows.values())
    by = {}
    for d in rows.values():
        step = step_of(d["name"], mode, sep)
        if step is None or "SQ_VALU_MFMA_BUSY_CYCLES" not in d:
            continue
        by.setdefault(step, []).append(d)
    out = [f"# MFMA use per launch: {workload} ({mode})", "",
           f"sources_digest: {kernel_sources_digest()}", "",
           "Command (from the repository root on the GPU host):", "", "```", command, "```", "",
           f"busy cycles per SIMD = SQ_VALU_MFMA_BUSY_CYCLES / {simds}; busy at {ghz} GHz = those "
           f"cycles at the nominal clock over the dispatch's duration (the fraction of the nominal "
           "bf16 peak the kernel reaches; the counter run serialises dispatches, so durations are "
           "a little longer than in the timed runs); bf16 GFLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x "
           f"512, what the MFMA units executed.  GRBM_GUI_ACTIVE / {xcds} covers the whole "
           "counter-collection window of a dispatch, not the kernel alone, so it is listed but not "
           "used as a clock.", "",
           "| step | dispatches | duration us | MFMA busy cycles per SIMD | busy at nominal clock | "
           "bf16 MFMA GFLOP per launch | GRBM_GUI_ACTIVE / XCDs |",
           "|---|---|---|---|---|---|---|"]
    for step in sorted(by):
        ds = by[step]
        n = len(ds)
        ns = sum(d["ns"] for d in ds) / n
        gui = sum(d.get("GRBM_GUI_ACTIVE", 0.0) for d in ds) / n / xcds
        busy = sum(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for d in ds) / n / simds
        flops = sum(d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for d in ds) / n * 512
        frac = busy / (ghz * ns) if ns > 0 else 0.0
        out.append(f"| {step} | {n} | {ns / 1e3:.2f} | {busy:.0f} | {100 * frac:.1f}% | "
                   f"{flops / 1e9:.2f} | {gui:.0f} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(prog="profsum")
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("--title", required=True)
    t.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--mode", choices=("decode", "prefill"), required=True)
    c.add_argument("--calib-bytes", type=int, required=True)
    c.add_argument("--fetch-command", required=True)
    c.add_argument("--write-command", required=True)
    f = sub.add_parser("mfma")
    f.add_argument("csv")
    f.add_argument("--workload", required=True)
    f.add_argument("--mode", choices=("decode", "prefill"), required=True)
    f.add_argument("--command", required=True)
    f.add_argument("--xcds", type=int, default=8)
    f.add_argument("--simds", type=int, default=1024)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        sys.stdout.write(trace_table(a.stats_csv, a.title, a.command))
    elif a.cmd == "mfma":
        sys.stdout.write(mfma_table(a.csv, a.workload, a.mode, a.command, a.xcds, a.simds))
    else:
        sys.stdout.write(counters_table(a.fetch, a.write, a.workload, a.mode, a.calib_bytes,
                                        a.fetch_command, a.write_command))


if __name__ == "__main__":
    main()
