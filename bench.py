"""Benchmark of the multi-LoRA batched linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one lora_linear call (segment build, shrink, base GEMM, expand) on one batch.
The headline workload is the decode batch of the Llama-2-7B q_proj geometry: x[64, 4096]
bf16, W[4096, 4096], 32 resident adapters of rank 16, one adapter id per row (uniform,
unsorted), alpha = 32.  Inputs are synthetic (seeded generator) and resident in HBM before
the timed region.  Each step uses the next of several device copies of (W, A, B) ("layers"),
enough to exceed the 256 MB Infinity Cache, so the weights stream from HBM as they would in a
forward pass over many layers.  Exactly K steps are captured as one HIP graph (checked
against an eager call of its last step) and replayed once between two synchronisations:
that replay gives `value` and `ms_per_step`.

Also reported, outside that timed region: the spread of further replays of the same graph
(p10 / p50 / p90 per step), single calls timed one by one with HIP events (cold: a 512 MiB
write evicts L2 and the Infinity Cache before each call; warm: the same call repeated), the
roofline of the dominant kernel (HIP-event duration per launch, algorithmic bytes or flops
per launch), the CPU oracle timed on the host on every workload, a per-kernel breakdown,
the other decode and prefill workloads under "workloads", the MoE-LoRA decode workload
(lora_moe_linear: 64 tokens routed top-4 over 32 experts of 2880 x 2880, 8 adapters of rank
16) under "moe" with its own roofline and oracle time, and three sweeps: step time
against the number of distinct adapters in a 64-row batch, against the adapters' rank, and
decode against prefill sequence over the batch size (where LORA_MODE_AUTO switches).
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
MALL_BYTES = 256 << 20       # Infinity Cache
ROTATE_BYTES = 640 << 20     # device bytes of weights cycled through per rotation

METRIC = "LoRA-linear tokens/s (decode & prefill, 4096²) + % HBM / MFMA peak"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------
# algorithmic work per kernel launch
# ---------------------------------------------------------------------------------------


def algorithmic_work(w, d_in: int, d_out: int, prefill: bool, y_bytes: int = 2) -> dict:
    """Bytes and flops the method must move / compute, per kernel of one call.

    Adapters count at their true rank and only when touched; x rows with an adapter are read
    once by the shrink; t is written once and read once (fp32); y is read and written once
    by the expand on LoRA rows.  The base GEMM reads W and x and writes y once.  Padded
    ranks, untouched adapters, id -1 rows and split-K partial sums are not counted.
    """
    ids, ranks = w.ids, w.ranks
    M = w.M
    lora = ids >= 0
    m_lora = int(lora.sum())
    touched = np.unique(ids[lora])
    r_touched = int(ranks[touched].sum()) if len(touched) else 0
    r_rows = int(ranks[ids[lora]].sum()) if m_lora else 0
    a_bytes = r_touched * d_in * 2
    b_bytes = r_touched * d_out * 2
    t_bytes = r_rows * 4
    shrink = a_bytes + m_lora * d_in * 2 + t_bytes
    expand = b_bytes + t_bytes + 2 * m_lora * d_out * y_bytes
    base_flops = 2.0 * M * d_in * d_out
    lora_flops = 2.0 * r_rows * (d_in + d_out)
    gemm_bytes = d_in * d_out * 2 + M * d_in * 2
    out = {
        "build_segments": {"bytes": 8 * M, "flops": 0.0},
        "shrink": {"bytes": shrink, "flops": 2.0 * r_rows * d_in},
        "shrink_finalize": {"bytes": 0, "flops": 0.0},
        "splitk_reduce": {"bytes": M * d_out * y_bytes, "flops": 0.0},
        "expand": {"bytes": expand, "flops": 2.0 * r_rows * d_out},
        "lora_bytes": shrink + expand,
        "call_flops": base_flops + lora_flops,
        "call_bytes": gemm_bytes + M * d_out * y_bytes + shrink + expand,
    }
    if prefill:
        out["gemm_prefill_lora"] = {"bytes": gemm_bytes + M * d_out * y_bytes,
                                    "flops": base_flops + 2.0 * r_rows * d_out}
    else:
        out["gemm_decode"] = {"bytes": gemm_bytes, "flops": base_flops}
        # small-batch decode path: one split-K GEMM over W and the touched A_i side by side
        # (x read; t leaves as split partials, not counted), then the ordered reduction with
        # the expand (the touched B_i, t read, y written once)
        out["decode_gemm_lora"] = {"bytes": gemm_bytes + a_bytes,
                                   "flops": base_flops + 2.0 * r_rows * d_in}
        # medium decode batches: the same GEMM without the shrink (W, x)
        out["decode_gemm"] = {"bytes": gemm_bytes, "flops": base_flops}
        # fp8 base: W8 (one byte per weight) + per-column scales + x
        out["decode_gemm_fp8"] = {"bytes": d_in * d_out + 4 * d_out + M * d_in * 2,
                                  "flops": base_flops}
        # fp8 base with the shrink as adapter tiles of the same launch (batches of <= 128 rows)
        out["decode_gemm_fp8_lora"] = {"bytes": d_in * d_out + 4 * d_out + M * d_in * 2 + a_bytes,
                                       "flops": base_flops + 2.0 * r_rows * d_in}
        out["decode_reduce_lora"] = {"bytes": b_bytes + t_bytes + M * d_out * y_bytes,
                                     "flops": 2.0 * r_rows * d_out}
    return out


# ---------------------------------------------------------------------------------------
# device setup
# ---------------------------------------------------------------------------------------


def _bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class DeviceLayers:
    """Device copies ("layers") of one projection's weights, cycled step by step.  With fp8,
    the base weight of every layer is fp8 E4M3 codes W8[d_out, d_in] plus column scales."""

    def __init__(self, w, pi, n_layers, rotate_x, torch, compact=False, fp8=False):
        p = w.projections[pi]
        self.d_in, self.d_out = p.d_in, p.d_out
        self.layers = []
        self.w_scale = None
        W_h = p.W
        if fp8:
            from synth import fp8_base

            W_h, ws_h = fp8_base(w.seed, p.d_in, p.d_out)
            self.w_scale = torch.from_numpy(ws_h).cuda()
        A_h, B_h = p.A, p.B
        self.off, self.pool_rows = None, 0
        if compact:  # the same adapters stored at their own rank (lora_linear_compact)
            from synth import compact_pool

            A_h, B_h, off, self.pool_rows = compact_pool(p.A, p.B, w.ranks)
            self.off = torch.from_numpy(off).cuda()
        x0 = _bf16(p.x, torch)
        for i in range(n_layers):
            W = torch.from_numpy(W_h).cuda() if fp8 else _bf16(W_h, torch)
            A = _bf16(A_h, torch)
            B = _bf16(B_h, torch)
            x = _bf16(p.x, torch) if (rotate_x and i > 0) else x0
            self.layers.append((x, W, A, B))


def split_group_kernels(ks, n):
    """Per-projection kernel lists of one lora_linear_multi call over n projections: a kernel
    name launched n times (every launch when the call ran projection by projection) goes to
    the projections in order; a launch shared by the group (the merged shrink, GEMM and
    reduction, the segment build) is split evenly between them."""
    out = [[] for _ in range(n)]
    names = [name for name, _ in ks]
    seen = {}
    for name, ms in ks:
        if names.count(name) == n:
            k = seen.get(name, 0)
            seen[name] = k + 1
            out[k].append((name, ms))
        else:
            for q in range(n):
                out[q].append((name, ms / n))
    return out


def layers_needed(w, rotate_x: bool, compact: bool = False, fp8: bool = False) -> int:
    per = 0
    for p in w.projections:
        pool = (int(w.ranks.sum()) * (p.d_in + p.d_out) * 2) if compact else p.A.nbytes + p.B.nbytes
        per += (p.W.nbytes // 2 if fp8 else p.W.nbytes) + pool + (p.x.nbytes if rotate_x else 0)
    return max(1, -(-ROTATE_BYTES // per))


class Runner:
    """One workload on the device: L layers, shared ids / ranks / scale, one output per
    projection, workspace; `step(i)` enqueues one step (all projections) for layer i % L."""

    def __init__(self, w, mode, torch, L, rotate_x=False, prebuilt_segments=False, compact=False,
                 fp8=False, merge=True):
        self.torch, self.w, self.mode, self.L = torch, w, mode, L
        self.compact, self.fp8 = compact, fp8
        self.M, self.n, self.r_max = w.M, w.n_adapters, w.r_max
        self.ids = torch.from_numpy(w.ids.astype(np.int32)).cuda()
        self.ranks = torch.from_numpy(w.ranks.astype(np.int32)).cuda()
        self.scale = torch.from_numpy((w.alpha / w.ranks.astype(np.float32)).astype(np.float32)).cuda()
        self.projs = [DeviceLayers(w, pi, L, rotate_x, torch, compact, fp8)
                      for pi in range(len(w.projections))]
        self.ys = [torch.empty((w.M, pr.d_out), dtype=torch.bfloat16, device="cuda") for pr in self.projs]
        # projections that read the same x with the same shape (an MLP's gate and up) run as one
        # lora_linear_multi call
        self.groups = []
        for pi, p in enumerate(w.projections):
            g = self.groups[-1] if self.groups else None
            q = w.projections[g[0]] if g else None
            if (merge and not (compact or fp8) and g and len(g) < L_.LORA_MAX_PROJ and p.x is q.x
                    and (p.d_in, p.d_out) == (q.d_in, q.d_out)):
                g.append(pi)
            else:
                self.groups.append([pi])
        nb = max(L_.lora_workspace_bytes(w.M, pr.d_in, pr.d_out, w.r_max, w.n_adapters) for pr in self.projs)
        for g in self.groups:
            if len(g) > 1:
                pr = self.projs[g[0]]
                nb = max(nb, L_.lora_workspace_bytes_multi(w.M, pr.d_in, pr.d_out, w.r_max,
                                                           w.n_adapters, len(g)))
        self.ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
        self.ws_bytes = nb
        self.segs = L_.Segments(w.M, w.n_adapters) if prebuilt_segments else None

    def _multi_args(self, g, li):
        pr = self.projs[g[0]]
        x = pr.layers[li][0]
        return (x, [self.projs[q].layers[li][1] for q in g], [self.projs[q].layers[li][2] for q in g],
                [self.projs[q].layers[li][3] for q in g], self.scale, self.ranks, self.ids, self.M,
                pr.d_in, pr.d_out, self.r_max, self.n, self.segs, [self.ys[q] for q in g],
                L_.LORA_BF16, self.mode, self.ws, self.ws_bytes)

    def step(self, i):
        li = i % self.L
        if self.segs is not None:
            L_.lora_build_segments(self.ids, self.M, self.n, self.segs)
        for g in self.groups:
            if len(g) > 1:
                L_.lora_linear_multi(*self._multi_args(g, li))
                continue
            pr, y = self.projs[g[0]], self.ys[g[0]]
            x, W, A, B = pr.layers[li]
            if self.fp8:
                L_.lora_linear_fp8w(x, W, pr.w_scale, A, B, self.scale, self.ranks, self.ids, self.M,
                                    pr.d_in, pr.d_out, self.r_max, self.n, self.segs, y,
                                    L_.LORA_BF16, self.mode, self.ws, self.ws_bytes)
                continue
            if self.compact:
                L_.lora_linear_compact(x, W, A, B, self.scale, self.ranks, pr.off, pr.pool_rows,
                                       self.ids, self.M, pr.d_in, pr.d_out, self.r_max, self.n,
                                       self.segs, y, L_.LORA_BF16, self.mode, self.ws,
                                       self.ws_bytes)
                continue
            L_.lora_linear(x, W, A, B, self.scale, self.ranks, self.ids, self.M, pr.d_in, pr.d_out,
                           self.r_max, self.n, self.segs, y, L_.LORA_BF16, self.mode, self.ws,
                           self.ws_bytes)

    def profile(self, i):
        """Per-kernel HIP-event durations of one step, queued behind two ordinary steps of other
        layers: the GPU is then busy as in the timed replays when the step's kernels start (after
        an idle GPU sleep the first kernel measured up to 15% longer than in the replays)."""
        li = i % self.L
        self.step(i + 1)
        self.step(i + 2)
        out = []
        if self.segs is not None:
            L_.lora_build_segments(self.ids, self.M, self.n, self.segs)
        for g in self.groups:
            if len(g) > 1:
                out.extend(split_group_kernels(L_.lora_linear_multi_profiled(*self._multi_args(g, li)),
                                               len(g)))
                continue
            pr, y = self.projs[g[0]], self.ys[g[0]]
            x, W, A, B = pr.layers[li]
            if self.fp8:
                ks = L_.lora_linear_fp8w_profiled(
                    x, W, pr.w_scale, A, B, self.scale, self.ranks, self.ids, self.M, pr.d_in,
                    pr.d_out, self.r_max, self.n, self.segs, y, L_.LORA_BF16, self.mode, self.ws,
                    self.ws_bytes)
            elif self.compact:
                ks = L_.lora_linear_compact_profiled(
                    x, W, A, B, self.scale, self.ranks, pr.off, pr.pool_rows, self.ids, self.M,
                    pr.d_in, pr.d_out, self.r_max, self.n, self.segs, y, L_.LORA_BF16, self.mode,
                    self.ws, self.ws_bytes)
            else:
                ks = L_.lora_linear_profiled(x, W, A, B, self.scale, self.ranks, self.ids, self.M,
                                             pr.d_in, pr.d_out, self.r_max, self.n, self.segs, y,
                                             L_.LORA_BF16, self.mode, self.ws, self.ws_bytes)
            out.append(ks)
        return out


def capture(runner, steps, torch):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        runner.step(0)  # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(steps):
            runner.step(i)
    torch.cuda.synchronize()
    return g


def check_graph_against_eager(runner, graph, torch, steps):
    """The graph's outputs equal an eager call of its last step, bit for bit."""
    graph.replay()
    torch.cuda.synchronize()
    from_graph = [y.clone() for y in runner.ys]
    runner.step(steps - 1)
    torch.cuda.synchronize()
    for a, b in zip(from_graph, runner.ys):
        if not torch.equal(a.view(torch.int16), b.view(torch.int16)):
            raise RuntimeError("graph replay differs from the eager call")


FLUSH_BYTES = 512 << 20  # more than L2 (8 x 4 MB) and the 256 MB Infinity Cache together


def pct(v, q):
    return float(np.percentile(np.asarray(v, np.float64), q))


def spread(v):
    return {"p10": pct(v, 10), "p50": pct(v, 50), "p90": pct(v, 90), "n": len(v)}


def per_call_times(runner, torch, reps):
    """Single calls (one step each, layer 0), each between two HIP events on the stream:
    cold (a FLUSH_BYTES write before each call, outside its events) and warm (the same call
    back to back).  Returns µs spreads."""
    g = capture(runner, 1, torch)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    out = {}
    for kind in ("cold", "warm"):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        g.replay()
        torch.cuda.synchronize()
        for e0, e1 in evs:
            if kind == "cold":
                flush.fill_(1)
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        out[kind] = {k: (v * 1e3 if k != "n" else v)
                     for k, v in spread([e0.elapsed_time(e1) for e0, e1 in evs]).items()}
    del g, flush
    return out


def measure(runner, steps, warmup, torch, profile_reps=20, replays=9, call_reps=100):
    """Timed graph replay of exactly `steps` steps, further replays for the spread, single
    calls cold and warm, plus per-kernel averages."""
    g = capture(runner, steps, torch)
    gw = capture(runner, max(1, warmup), torch) if warmup > 0 else None
    check_graph_against_eager(runner, g, torch, steps)
    if gw is not None:
        gw.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    # the spread over further replays of the same graph (ms per step)
    per_step = []
    for _ in range(replays):
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        per_step.append(ev0.elapsed_time(ev1) / steps)
    # eager steps, for reference (host launch cost included)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_eager = min(steps, 50)
    for i in range(n_eager):
        runner.step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t1) * 1e3 / n_eager
    del g, gw
    calls = per_call_times(runner, torch, call_reps) if call_reps > 0 else None
    # per-kernel durations
    sums, counts = {}, {}
    for i in range(profile_reps):
        for pi, ks in enumerate(runner.profile(i)):
            for name, ms in ks:
                key = (pi, name)
                sums[key] = sums.get(key, 0.0) + ms
                counts[key] = counts.get(key, 0) + 1
    kernels = {k: sums[k] / counts[k] for k in sums}
    return ms_total, wall, eager_ms, kernels, spread(per_step), calls


# ---------------------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------------------


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS when that is
    set (the host's CPU share on a shared machine)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    return min(n, int(env)) if env.isdigit() and int(env) > 0 else n


def oracle_call_s(w, threads: int, reps: int) -> float:
    """Median wall time of `reps` oracle calls over every projection of w (inputs already
    widened to fp32, outside the timing)."""
    import oracle
    from synth import bf16_bits_to_f32

    ps = [tuple(bf16_bits_to_f32(v) for v in (p.x, p.W, p.A, p.B)) for p in w.projections]
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        for xf, Wf, Af, Bf in ps:
            oracle.lora_linear(xf, Wf, Af, Bf, w.alpha, w.ranks, w.ids, n_threads=threads)
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_baseline(w, seconds: float, all_workloads=None):
    """The oracle on the host: the headline workload for about `seconds` (the reported
    value), then every workload once or three times on all allowed threads, and the small
    ones on one thread."""
    import oracle
    from synth import bf16_bits_to_f32

    p = w.projections[0]
    xf, Wf, Af, Bf = (bf16_bits_to_f32(v) for v in (p.x, p.W, p.A, p.B))
    threads = host_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.lora_linear(xf, Wf, Af, Bf, w.alpha, w.ranks, w.ids, n_threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    out = {"value": w.M * reps / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"the full {w.M}-row batch of {w.name}, {reps} oracle calls in {el:.1f} s "
                     f"(plain C fp32 row loop, OpenMP over rows)",
           "cpu_model": cpu_model(), "host_cpu_count": os.cpu_count()}
    per = {}
    for name, wl in (all_workloads or {}).items():
        small = wl.M * sum(q.d_in * q.d_out for q in wl.projections) <= 256 * 4096 * 4096
        entry = {}
        for th in ((threads, 1) if small else (threads,)):
            sec = oracle_call_s(wl, th, 3 if small else 1)
            entry[f"threads_{th}"] = {"s_per_call": sec, "tokens_per_s": wl.M / sec}
        per[name] = entry
    if per:
        out["per_workload"] = per
    return out


# ---------------------------------------------------------------------------------------
# traffic from committed rocprofv3 counter summaries
# ---------------------------------------------------------------------------------------


def committed_traffic(workload: str, kernel: str):
    """HBM bytes per launch from profiles/counters_<workload>.md, if taken on these sources."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    from profsum import kernel_sources_digest

    m = re.search(r"sources_digest:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_sources_digest():
        return None
    m = re.search(rf"^traffic\s+{re.escape(kernel)}\s+([0-9.eE+]+)", text, re.M)
    return float(m.group(1)) if m else None


# ---------------------------------------------------------------------------------------


def roofline_for(name, ms, work, workload):
    wk = work[name]
    if name.startswith("gemm_prefill"):
        achieved = wk["flops"] / (ms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        achieved = wk["bytes"] / (ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    r["frac"] = r["achieved"] / r["peak"]
    r["kernel"] = name
    r["us_per_launch"] = ms * 1e3
    r["algorithmic_per_launch"] = wk["flops"] if r["bound"] == "mfma" else wk["bytes"]
    r["traffic"] = committed_traffic(workload, name)
    return r


def summarize(w, runner, ms_total, steps, wall, eager_ms, kernels, prefill):
    projs = w.projections
    per_proj = []
    lora_s = base_s = 0.0
    lora_bytes = 0
    total_kernel_ms = 0.0
    for pi, p in enumerate(projs):
        work = algorithmic_work(w, p.d_in, p.d_out, prefill)
        ks = {name: ms for (qi, name), ms in kernels.items() if qi == pi}
        total_kernel_ms += sum(ks.values())
        entry = {"projection": p.name, "d_in": p.d_in, "d_out": p.d_out,
                 "kernels_us": {k: round(v * 1e3, 2) for k, v in ks.items()}}
        gname = "gemm_prefill_lora" if prefill else (
            "decode_gemm_lora" if "decode_gemm_lora" in ks else
            "decode_gemm_fp8_lora" if "decode_gemm_fp8_lora" in ks else
            "decode_gemm_fp8" if "decode_gemm_fp8" in ks else
            "decode_gemm" if "decode_gemm" in ks else "gemm_decode")
        if gname in ks:
            g_ms = ks[gname]
            entry["gemm_tflops"] = work[gname]["flops"] / (g_ms * 1e-3) / 1e12
            entry["gemm_mfma_frac"] = entry["gemm_tflops"] / BF16_PEAK_TFLOPS
            entry["gemm_gbs"] = work[gname]["bytes"] / (g_ms * 1e-3) / 1e9
            entry["gemm_hbm_frac"] = entry["gemm_gbs"] / HBM_PEAK_GBS
            base_s += (g_ms + ks.get("splitk_reduce", 0.0)) * 1e-3
        lk = [k for k in ("shrink", "shrink_finalize", "expand") if k in ks]
        if not prefill and lk and "expand" in ks:
            l_ms = sum(ks[k] for k in lk)
            entry["shrink_expand_us"] = l_ms * 1e3
            entry["shrink_expand_gbs"] = work["lora_bytes"] / (l_ms * 1e-3) / 1e9
            entry["shrink_expand_hbm_frac"] = entry["shrink_expand_gbs"] / HBM_PEAK_GBS
            lora_bytes += work["lora_bytes"]
        elif not prefill and "shrink" in ks and "decode_reduce_lora" in ks:
            # medium and stream-K decode paths: the shrink, then the pass that adds the GEMM's
            # partial sums and the expand (its bytes: B_i, t, y written once)
            l_ms = sum(ks[k] for k in ("shrink", "shrink_finalize", "decode_reduce_lora") if k in ks)
            l_bytes = work["shrink"]["bytes"] + work["decode_reduce_lora"]["bytes"]
            entry["shrink_reduce_lora_us"] = l_ms * 1e3
            entry["shrink_reduce_lora_gbs"] = l_bytes / (l_ms * 1e-3) / 1e9
            entry["shrink_reduce_lora_hbm_frac"] = entry["shrink_reduce_lora_gbs"] / HBM_PEAK_GBS
        lora_s += sum(ks.get(k, 0.0) for k in ("build_segments", "shrink", "shrink_finalize", "expand")) * 1e-3
        per_proj.append(entry)
    ms_step = ms_total / steps
    return {
        "tokens_per_s": w.M * steps / (ms_total * 1e-3),
        "ms_per_step": ms_step,
        "ms_per_step_eager": eager_ms,
        "kernel_sum_ms": total_kernel_ms,
        # segment path only: the small-batch path overlaps the shrink with the GEMM
        "lora_overhead_vs_base_gemm": (lora_s / base_s) if base_s > 0 and lora_s > 0 else None,
        "projections": per_proj,
    }


def base_only_ms(w, runner, steps, torch):
    """ms per step of the same launches with every id = -1 (no row has an adapter): what
    this path costs for the bare base model, to compare the LoRA step against."""
    keep = runner.ids
    runner.ids = torch.full_like(keep, -1)
    try:
        g = capture(runner, steps, torch)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        del g
    finally:
        runner.ids = keep
    return ms


_WORKLOADS = {}


def workload(config):
    from synth import make_workload

    if config not in _WORKLOADS:
        _WORKLOADS[config] = make_workload(config).as_bf16()
    return _WORKLOADS[config]


def run_workload(config, mode_name, steps, warmup, torch, profile_reps=20, compact=False,
                 call_reps=100, fp8=False, merge=True):
    w = workload(config)
    prefill = mode_name == "prefill"
    mode = L_.LORA_MODE_PREFILL if prefill else L_.LORA_MODE_DECODE
    rotate_x = prefill
    L = layers_needed(w, rotate_x, compact, fp8)
    runner = Runner(w, mode, torch, L, rotate_x=rotate_x, prebuilt_segments=len(w.projections) > 1,
                    compact=compact, fp8=fp8, merge=merge)
    log(f"bench: {w.name} mode={mode_name} layers={L} steps={steps} compact={compact} fp8={fp8}")
    ms_total, wall, eager_ms, kernels, reps, calls = measure(runner, steps, warmup, torch,
                                                             profile_reps, call_reps=call_reps)
    s = summarize(w, runner, ms_total, steps, wall, eager_ms, kernels, prefill)
    s.update({"workload": w.name, "mode": mode_name, "layers_rotated": L, "steps": steps,
              "pool": "rank-compact (lora_linear_compact)" if compact else "padded to r_max",
              "base": "fp8 E4M3 W8[d_out, d_in] + column scales (lora_linear_fp8w)" if fp8 else "bf16 W",
              "ms_per_step_replays": reps, "us_per_call": calls,
              "merged_projections": [[w.projections[q].name for q in g] for g in runner.groups
                                     if len(g) > 1]})
    base_ms = base_only_ms(w, runner, steps, torch)
    s["base_only_ms_per_step"] = base_ms
    s["lora_overhead_vs_base_only"] = s["ms_per_step"] / base_ms - 1.0
    del runner
    return w, s, kernels, steps, ms_total


# ---------------------------------------------------------------------------------------
# MoE-LoRA
# ---------------------------------------------------------------------------------------


def moe_work(w, y_bytes: int = 2) -> dict:
    """Algorithmic bytes / flops of one lora_moe_linear call (per kernel).  Counted once:
    W[e] of every expert some slot is routed to, A[i][e] and B[i][e] of every (adapter,
    expert) pair some token uses (at the adapter's true rank), x, y (every slot row).  Split
    partial sums are not counted."""
    E, M, K, N = w.n_experts, w.M, w.d_in, w.d_out
    topk = w.topk_ids
    routed = topk >= 0
    active = np.unique(topk[routed])
    pairs = set()
    r_rows = 0
    for m in range(M):
        i = int(w.ids[m])
        for e in topk[m][topk[m] >= 0]:
            if i >= 0:
                pairs.add((i, int(e)))
                r_rows += int(w.ranks[i])
    r_pairs = sum(int(w.ranks[i]) for i, _ in pairs)
    n_routed = int(routed.sum())
    w_bytes = len(active) * K * N * 2
    a_bytes = r_pairs * K * 2
    b_bytes = r_pairs * N * 2
    x_bytes = M * K * 2
    y_out = M * w.top_k * N * y_bytes
    base_flops = 2.0 * n_routed * K * N
    return {
        "moe_gemm": {"bytes": w_bytes + a_bytes + x_bytes, "flops": base_flops + 2.0 * r_rows * K},
        "moe_reduce": {"bytes": b_bytes + y_out, "flops": 2.0 * r_rows * N},
        "call_bytes": w_bytes + a_bytes + b_bytes + x_bytes + y_out,
        "active_experts": int(len(active)), "adapter_expert_pairs": len(pairs),
        "routed_slots": n_routed,
    }


class MoeRunner:
    """The MoE workload on the device: L copies of (W, A, B) cycled step by step (more bytes
    than the Infinity Cache), shared routing and ids; `step(i)` = one lora_moe_linear call."""

    def __init__(self, w, torch, L):
        self.torch, self.w, self.L = torch, w, L
        self.layers = [(_bf16(w.W, torch), _bf16(w.A, torch), _bf16(w.B, torch)) for _ in range(L)]
        self.x = _bf16(w.x, torch)
        self.ids = torch.from_numpy(w.ids.astype(np.int32)).cuda()
        self.ranks = torch.from_numpy(w.ranks.astype(np.int32)).cuda()
        self.scale = torch.from_numpy((w.alpha / w.ranks.astype(np.float32)).astype(np.float32)).cuda()
        self.topk = torch.from_numpy(w.topk_ids.astype(np.int32)).cuda()
        self.topk_w = torch.from_numpy(w.topk_w.astype(np.float32)).cuda()
        self.ys = [torch.empty((w.M, w.top_k, w.d_out), dtype=torch.bfloat16, device="cuda")]
        self.ws, self.ws_bytes = L_.moe_workspace(w.M, w.top_k, w.n_experts, w.d_in, w.d_out,
                                                  w.r_max, w.n_adapters)

    def _args(self, i):
        W, A, B = self.layers[i % self.L]
        w = self.w
        return (self.x, W, A, B, self.scale, self.ranks, self.ids, self.topk, self.topk_w, w.M,
                w.top_k, w.n_experts, w.d_in, w.d_out, w.r_max, w.n_adapters, self.ys[0],
                L_.LORA_BF16, L_.LORA_MODE_DECODE, self.ws, self.ws_bytes)

    def step(self, i):
        L_.lora_moe_linear(*self._args(i))

    def profile(self, i):
        # queued behind two ordinary calls of other layers (see Runner.profile)
        self.step(i + 1)
        self.step(i + 2)
        return [L_.lora_moe_linear_profiled(*self._args(i))]


def moe_layers_needed(w) -> int:
    per = w.W.nbytes + w.A.nbytes + w.B.nbytes
    return max(2, -(-ROTATE_BYTES // per))


def run_moe(steps, warmup, torch, profile_reps=20, call_reps=50):
    """The MoE decode workload: graph of `steps` calls, spread, single calls, per-kernel
    durations, the same calls with every id -1, the roofline of the routed GEMM."""
    from synth import make_moe_workload

    w = make_moe_workload()
    L = moe_layers_needed(w)
    runner = MoeRunner(w, torch, L)
    log(f"bench: {w.name} layers={L} steps={steps}")
    ms_total, wall, eager_ms, kernels, reps, calls = measure(runner, steps, warmup, torch,
                                                             profile_reps, call_reps=call_reps)
    ks = {name: ms for (_, name), ms in kernels.items()}
    work = moe_work(w)
    ms_step = ms_total / steps
    keep = runner.ids
    runner.ids = torch.full_like(keep, -1)
    try:
        g = capture(runner, steps, torch)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        base_ms = ev0.elapsed_time(ev1) / steps
        del g
    finally:
        runner.ids = keep
    g_ms = ks.get("moe_gemm")
    roof = None
    if g_ms:
        achieved = work["moe_gemm"]["bytes"] / (g_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "kernel": "moe_gemm", "us_per_launch": g_ms * 1e3,
                "algorithmic_per_launch": work["moe_gemm"]["bytes"],
                "traffic": committed_traffic(w.name, "moe_gemm")}
    out = {
        "workload": w.name, "M": w.M, "top_k": w.top_k, "n_experts": w.n_experts,
        "d_in": w.d_in, "d_out": w.d_out, "n_adapters": w.n_adapters, "r_max": w.r_max,
        "layers_rotated": L, "steps": steps,
        "tokens_per_s": w.M * steps / (ms_total * 1e-3),
        "ms_per_step": ms_step, "ms_per_step_eager": eager_ms,
        "ms_per_step_replays": reps, "us_per_call": calls,
        "kernels_us": {k: round(v * 1e3, 2) for k, v in ks.items()},
        "base_only_ms_per_step": base_ms,
        "lora_overhead_vs_base_only": ms_step / base_ms - 1.0,
        "call_hbm_frac": work["call_bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic": {k: v for k, v in work.items() if not isinstance(v, dict)},
        "roofline": roof,
    }
    del runner
    torch.cuda.empty_cache()
    return w, out


def moe_cpu_baseline(w, threads: int, seconds: float = 3.0):
    """The oracle's MoE layer on the host: full-batch calls for about `seconds` (inputs
    widened to fp32 outside the timing)."""
    import oracle
    from synth import bf16_bits_to_f32

    xf, Wf, Af, Bf = (bf16_bits_to_f32(v) for v in (w.x, w.W, w.A, w.B))
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.moe_lora_linear(xf, Wf, Af, Bf, w.alpha, w.ranks, w.ids, w.topk_ids, w.topk_w,
                               n_threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": w.M * reps / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the full {w.M}-token batch of {w.name}, {reps} oracle calls in {el:.1f} s"}


# ---------------------------------------------------------------------------------------
# sweeps
# ---------------------------------------------------------------------------------------


def step_ms(w, mode, torch, steps, rotate_x=False):
    """ms per step of one graph of `steps` steps (weights rotated as in the workloads), and
    the same with every id = -1."""
    L = layers_needed(w, rotate_x)
    runner = Runner(w, mode, torch, L, rotate_x=rotate_x)
    g = capture(runner, steps, torch)
    g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(3):
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        ts.append(ev0.elapsed_time(ev1) / steps)
    del g
    base = base_only_ms(w, runner, steps, torch)
    del runner
    torch.cuda.empty_cache()
    return float(np.median(ts)), base


def sweeps(torch, steps=32):
    """Decode q_proj geometry (x[64, 4096], W[4096, 4096]) with a varied adapter count and
    rank, and decode vs prefill sequence over the batch size.  Inputs: synth.random_case."""
    from synth import random_case

    out = {"adapters": [], "rank": [], "auto_threshold": []}
    M, d = 64, 4096
    rng = np.random.default_rng(7)
    for T in (1, 2, 4, 8, 16, 32, 64):  # distinct adapters among the 64 rows (pool of 128, r 16)
        ids = rng.permutation(np.arange(M) % T).astype(np.int32)
        w = random_case(500 + T, M, d, d, 128, 16, ranks=[16] * 128, ids=ids, base_frac=0.0)
        ms, base = step_ms(w, L_.LORA_MODE_DECODE, torch, steps)
        out["adapters"].append({"distinct_adapters": T, "ms_per_step": ms, "base_only_ms": base,
                                "lora_overhead_vs_base_only": ms / base - 1.0})
        log(f"sweep: adapters {T}: {ms * 1e3:.2f} us")
    for r in (8, 16, 32, 64):  # 32 adapters of rank r, uniform ids
        w = random_case(600 + r, M, d, d, 32, r, ranks=[r] * 32, base_frac=0.0)
        ms, base = step_ms(w, L_.LORA_MODE_DECODE, torch, steps)
        out["rank"].append({"rank": r, "distinct_adapters": int(len(np.unique(w.ids))),
                            "ms_per_step": ms, "base_only_ms": base,
                            "lora_overhead_vs_base_only": ms / base - 1.0})
        log(f"sweep: rank {r}: {ms * 1e3:.2f} us")
    for m in (256, 512, 768, 1024, 1536, 2048):  # 8 adapters of rank 16, runs of M/8 rows
        ids = np.repeat(np.arange(8), m // 8).astype(np.int32)
        w = random_case(700 + m, m, d, d, 8, 16, ranks=[16] * 8, ids=ids, base_frac=0.0)
        dec, _ = step_ms(w, L_.LORA_MODE_DECODE, torch, 8, rotate_x=True)
        pre, _ = step_ms(w, L_.LORA_MODE_PREFILL, torch, 8, rotate_x=True)
        out["auto_threshold"].append({"M": m, "decode_ms": dec, "prefill_ms": pre})
        log(f"sweep: M {m}: decode {dec * 1e3:.1f} us, prefill {pre * 1e3:.1f} us")
    faster = [e["M"] for e in out["auto_threshold"] if e["prefill_ms"] < e["decode_ms"]]
    out["prefill_faster_from_rows"] = min(faster) if faster else None
    out["lora_prefill_min_rows"] = L_.LORA_PREFILL_MIN_ROWS
    return out


CALIB_BYTES = 256 << 20


def pmc_pass(config, mode_name, steps, torch, compact=False, moe=False):
    """Eager steps of one workload, then the counter calibration kernel: torch.neg over
    CALIB_BYTES of bf16 (reads CALIB_BYTES, writes CALIB_BYTES), three times.  Meant to run
    under ``rocprofv3 --pmc``; no timing."""
    from synth import make_moe_workload, make_workload

    if moe:
        w = make_moe_workload()
        L = moe_layers_needed(w)
        runner = MoeRunner(w, torch, L)
    else:
        w = make_workload(config).as_bf16()
        prefill = mode_name == "prefill"
        mode = L_.LORA_MODE_PREFILL if prefill else L_.LORA_MODE_DECODE
        L = layers_needed(w, prefill, compact)
        runner = Runner(w, mode, torch, L, rotate_x=prefill,
                        prebuilt_segments=len(w.projections) > 1, compact=compact)
    for i in range(steps):
        runner.step(i)
    torch.cuda.synchronize()
    src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_pass": w.name, "mode": mode_name, "compact": compact, "steps": steps,
                      "layers_rotated": L,
                      "calibration": {"kernel": "torch.neg bf16", "bytes_read": CALIB_BYTES,
                                      "bytes_written": CALIB_BYTES, "launches": 3}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=5.0,
                    help="seconds of oracle calls on the headline workload (0: no CPU baseline)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other workloads, the sweeps and the per-workload CPU runs")
    ap.add_argument("--no-sweeps", action="store_true", help="skip the sweeps")
    ap.add_argument("--workload", type=int, default=2, choices=(2, 3, 4, 5),
                    help="workload of the headline line (2 = decode q_proj, the default)")
    ap.add_argument("--mode", default="decode", choices=("decode", "prefill"))
    ap.add_argument("--compact", action="store_true",
                    help="serve the headline (or --pmc-pass) workload from its rank-compact pool "
                         "(lora_linear_compact)")
    ap.add_argument("--moe", action="store_true",
                    help="only the MoE-LoRA decode workload (its own JSON line; with --pmc-pass, "
                         "its counter pass)")
    ap.add_argument("--separate-projections", action="store_true",
                    help="call lora_linear per projection also where projections share x (the "
                         "MLP's gate and up), instead of one lora_linear_multi call")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="only eager steps of the chosen workload plus the counter calibration "
                         "kernel, for rocprofv3 --pmc runs (FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the library runs "
              "on a single MI355X; sharding across GPUs is not implemented).", file=sys.stderr)
        sys.exit(2)

    import torch

    global L_
    from rank_adapter_gemm_sgmv_amd import lora as L_

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.pmc_pass:
        pmc_pass(args.workload, args.mode, args.steps, torch, args.compact, args.moe)
        return
    if args.moe:
        mw, moe = run_moe(args.steps, args.warmup, torch)
        print(json.dumps({"moe": moe, "cpu_baseline": moe_cpu_baseline(mw, host_threads(), args.cpu_seconds)
                          if args.cpu_seconds > 0 else None}), flush=True)
        return

    # headline: decode, q_proj geometry (unless another workload is asked for)
    w, head, kernels, steps, ms_total = run_workload(args.workload, args.mode, args.steps,
                                                     args.warmup, torch, compact=args.compact,
                                                     merge=not args.separate_projections)
    p0 = w.projections[0]
    work = algorithmic_work(w, p0.d_in, p0.d_out, args.mode == "prefill")
    kmain = {name: ms for (pi, name), ms in kernels.items() if pi == 0}
    dom = max(kmain, key=lambda k: kmain[k])
    roof = roofline_for(dom, kmain[dom], work, w.name + ("_compact" if args.compact else ""))

    workloads = {}
    if not args.headline_only:
        for cfg, mode_name, st, var in ((3, "decode", 128, ""), (3, "decode", 128, "compact"),
                                        (4, "prefill", 40, ""), (5, "decode", 64, ""),
                                        (5, "decode", 64, "separate-projections"),
                                        (4, "decode", 20, ""), (2, "prefill", 64, ""),
                                        (2, "decode", 128, "fp8base")):
            try:
                _, s, _, _, _ = run_workload(cfg, mode_name, st, 4, torch, profile_reps=8,
                                             compact=var == "compact", fp8=var == "fp8base",
                                             merge=var != "separate-projections")
                workloads[f"{s['workload']}:{mode_name}{'-' + var if var else ''}"] = s
            except Exception as e:  # report, do not hide the headline
                workloads[f"config{cfg}:{mode_name}"] = {"error": repr(e)}
            torch.cuda.empty_cache()

    moe = None
    if not args.headline_only:
        try:
            mw, moe = run_moe(64, 4, torch, profile_reps=8, call_reps=20)
            if args.cpu_seconds > 0:
                moe["cpu_baseline"] = moe_cpu_baseline(mw, host_threads(), min(args.cpu_seconds, 3.0))
        except Exception as e:  # report, do not hide the headline
            moe = {"error": repr(e)}
        torch.cuda.empty_cache()

    sw = None
    if not args.headline_only and not args.no_sweeps:
        try:
            sw = sweeps(torch)
        except Exception as e:  # report, do not hide the headline
            sw = {"error": repr(e)}
        torch.cuda.empty_cache()

    cpu = None
    if args.cpu_seconds > 0:
        others = None if args.headline_only else {workload(c).name: workload(c) for c in (1, 2, 3, 4, 5)}
        cpu = cpu_baseline(w, args.cpu_seconds, others)

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "d_in": p0.d_in, "d_out": p0.d_out,
                   "n_adapters": w.n_adapters, "r_max": w.r_max, "mode": args.mode,
                   "layers_rotated": head["layers_rotated"],
                   "timed_as": "one HIP graph of exactly the K steps, replayed once",
                   "pool": head["pool"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "spread": {"ms_per_step_replays": head["ms_per_step_replays"],
                   "us_per_call": head["us_per_call"]},
        "headline_detail": head,
        "workloads": workloads,
        "moe": moe,
        "sweeps": sw,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
