"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m rank_adapter_gemm_sgmv_amd.profsum trace STATS_CSV --title T --command C
        kernel-trace statistics (``rocprofv3 --kernel-trace --stats --output-format csv``)
        as a markdown table.

    python -m rank_adapter_gemm_sgmv_amd.profsum counters --fetch CSV --write CSV \
            --workload NAME --mode decode|prefill --calib-bytes N --fetch-command C --write-command C
        HBM traffic per launch of each kernel of the path, from two ``rocprofv3 --pmc`` runs
        of ``bench.py --pmc-pass`` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Both
        counters are scaled by what they read for the calibration kernel at the end of the
        pass, a plain elementwise kernel (torch.neg on bf16) that reads N bytes and writes N
        bytes: traffic = FETCH_SIZE * 1024 * N / FETCH_calib + WRITE_SIZE * 1024 * N / WRITE_calib.
        The output carries the digest of the kernel sources it was taken on; bench.py reports
        the traffic only while the sources still have that digest.
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
    ("reduce_lora_kernel", "decode_reduce_lora"),
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
]
_CALIB = "neg_kernel"


def kernel_sources_digest() -> str:
    """sha256 (16 hex digits) over the names and bytes of csrc/*.hip, *.h, *.cpp."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "csrc")
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


def trace_table(stats_csv: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    out = [f"# {title}", "", "Command (from the repository root on the GPU host):", "", "```",
           command, "```", "", "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
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
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        sys.stdout.write(trace_table(a.stats_csv, a.title, a.command))
    else:
        sys.stdout.write(counters_table(a.fetch, a.write, a.workload, a.mode, a.calib_bytes,
                                        a.fetch_command, a.write_command))


if __name__ == "__main__":
    main()
