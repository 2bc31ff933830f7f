#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet layer on one MI355X.

One step = one pass of the whole hot path on resident HBM inputs:
  * a chunked prefill of one 4096-token sequence (HK=16 query/key heads, HV=32
    value heads, d=128, bf16 q/k/v/out, fp32 gates and state, chunk 64, zero
    initial state, final state written), and
  * one decode step for a batch of 64 sequences against resident fp32 states
    (bf16 q/k/v/gates/out).
value = (4096 + 64) tokens per step / step time (tokens/s per layer); the
prefill and decode parts are also reported on their own.

Inputs are synthetic (gdn_synth). Several copies of every buffer set are
rotated through so that each step reads its state and inputs from HBM rather
than from the 256 MB Infinity Cache left warm by the previous step.

Timing: HIP events on the stream the library launches on (torch's current
stream), around exactly --steps steps after --warmup untimed steps, with
torch.cuda.synchronize() on both sides. Measurement passes of the same steps
run just before them: one brackets every step with events (the spread), then
prefill-only and decode-only rates, then one brackets every kernel launch
with the library's own event pairs (gdn_timing_start/stop: each kernel's
mean duration for the roofline). The parity check's GPU step runs first; the oracle it is
compared with (and the CPU baseline) runs after the timed region, so that the
GPU does not idle for its ~20 s right before the timed steps.

Output: one JSON line (see the "roofline" and "cpu_baseline" objects).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HK, HV, D, CHUNK = 16, 32, 128, 64
T_PREFILL, B_DECODE = 4096, 64
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "GDN layer tokens/s (prefill T=4K; decode B=64) + % MFMA / % HBM peak"


def scan_flops_per_token(hv=HV, dk=D, dv=D, c=CHUNK):
    """Algorithmic MFMA flops of the chunk-recurrent scan kernel per token:
    per value head K S^T, Q S^T, K^T (delta U) (each 2*dk*dv per token) and
    T Y, P U (each 2*C*dv per token)."""
    return hv * (6 * dk * dv + 4 * c * dv)


def prep_flops_per_token(hk=HK, hv=HV, dk=D, c=CHUNK):
    """Algorithmic MFMA flops of the chunk-preparation kernel per token:
    K K^T and Q K^T per query/key head (2*C*dk each), and W = T diag(b gamma) K
    per value head (2*C*dk)."""
    return hk * 4 * c * dk + hv * 2 * c * dk


def decode_bytes_per_step(b=B_DECODE, hk=HK, hv=HV, dk=D, dv=D, state_bytes=4):
    """Algorithmic HBM bytes of one decode step: the state (fp32, or bf16 with
    state_bytes=2) read and written once, bf16 q, k (per q/k head), v, gates
    and output."""
    return (b * hv * dv * dk * state_bytes * 2 + b * (2 * hk * dk + hv * dv) * 2 + b * hv * 2 * 2
            + b * hv * dv * 2)


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and whitespace are dropped,
    so that counters taken on the same code stay valid after a comment edit."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_deltanet_linear_02_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8", errors="replace") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode() + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from committed counter runs, if they were taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


KERNELS = {"schedule": "gdn_schedule_kernel", "prep": "gdn_prep_kernel", "scan": "gdn_scan_kernel",
           "decode": "gdn_decode_kernel", "token_scan": "gdn_token_scan_kernel",
           "decode_norm": "gdn_decode_norm_kernel", "norm_apply": "gdn_norm_apply_kernel"}


def _short_kernel(name: str) -> str:
    for short, key in KERNELS.items():
        if key in name:
            return short
    return "copy" if "copy" in name.lower() else "other"


def _template_ints(name: str) -> list:
    """The integer template arguments of a kernel name as rocprofv3 prints it
    (mangled, or demangled with the arguments between < and >)."""
    import re
    m = re.search(r"_kernelI(.*?)EEv", name)
    if m:
        return [int(x) for x in re.findall(r"Li(\d+)E", m.group(1) + "E")]
    m = re.search(r"_kernel<([^()]*)>\(", name)
    if m:
        return [int(x) for x in (a.strip() for a in m.group(1).split(",")) if x.isdigit()]
    return []


def _kernel_label(name: str) -> str:
    """Kernel name for the summaries, with the variant where a kernel has
    several: chunk size and state rows per workgroup (scan), chunk size
    (prep), state rows per lane group (token scan)."""
    short = _short_kernel(name)
    label = KERNELS.get(short, name)
    ints = _template_ints(name)
    if short == "scan" and len(ints) >= 3:
        norm = "Lb1E" in name or ", true>" in name
        label += f" (C={ints[0]}, {ints[-1]}-row slices{', norm fused' if norm else ''})"
    elif short == "prep" and ints:
        label += f" (C={ints[0]})"
    elif short == "token_scan" and len(ints) >= 3 and ints[-1] > 1:
        label += f" ({ints[-1]} rows per lane group)"
    return label


def _state_key(name: str) -> str:
    """Short kernel name, with "/bf16" appended for decode kernels built for
    bf16 state storage (their third template argument)."""
    import re
    short = _short_kernel(name)
    m = re.search(r"gdn_decode(?:_norm)?_kernelI(?:DF16b|f)(?:DF16b|f)(DF16b|f)Li", name)
    return short + "/bf16" if m and m.group(1) == "DF16b" else short


def _counter_means(directory: str, counter: str, probe_bytes: int, key=None):
    """Mean counter value (KiB) per dispatch of each library kernel, and the
    factor that maps the counter to bytes, taken from the probe copies (the
    dispatches of a copy kernel within 10% of the largest one)."""
    import csv
    key = key or _short_kernel
    path = os.path.join(directory, "run_counter_collection.csv")
    per = {}
    copies = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            short = key(r["Kernel_Name"])
            val = float(r["Counter_Value"])
            if short == "copy":
                copies.append(val)
            elif short != "other":
                per.setdefault(short, []).append(val)
    top = max(copies) if copies else 0.0
    probe = [c for c in copies if c >= 0.9 * top]
    if not probe:
        raise SystemExit(f"no probe copy found in {path}")
    kib = sum(probe) / len(probe)
    factor = probe_bytes / kib
    return {k: sum(v) / len(v) for k, v in per.items()}, factor, kib


def summarize_profiles(stats_dir: str, fetch_dir: str, write_dir: str, probe_mib: int):
    """Write profiles/traffic.json and the markdown summaries from rocprofv3
    runs of this script (kernel trace with --stats; one --pmc FETCH_SIZE and
    one --pmc WRITE_SIZE pass, each with --copy-probe-mib)."""
    import csv
    probe_bytes = probe_mib << 20
    fetch, ffac, fkib = _counter_means(fetch_dir, "FETCH_SIZE", probe_bytes)
    write, wfac, wkib = _counter_means(write_dir, "WRITE_SIZE", probe_bytes)
    h = kernel_source_hash()
    rd = _probe_check(fetch_dir, "FETCH_SIZE", ffac, probe_bytes, "reduce_kernel")
    wr = _probe_check(write_dir, "WRITE_SIZE", wfac, probe_bytes, "FillFunctor")
    traffic = {"source_hash": h, "probe_copy_bytes": probe_bytes,
               "fetch_bytes_per_kib": ffac, "write_bytes_per_kib": wfac,
               "check_read_only_sum_fetch_ratio": rd, "check_write_only_fill_write_ratio": wr}
    for short in ("schedule", "prep", "scan", "decode"):
        if short in fetch and short in write:
            fb, wb = fetch[short] * ffac, write[short] * wfac
            traffic[KERNELS[short]] = {"source_hash": h, "bytes_per_launch": fb + wb,
                                       "fetch_bytes": fb, "write_bytes": wb,
                                       "fetch_kib_raw": fetch[short], "write_kib_raw": write[short]}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    rows = []
    with open(os.path.join(stats_dir, "run_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append(r)
    lines = [
        "# Kernel time and HBM traffic: prefill 1x4096 + decode batch 64 (HK=16, HV=32, d=128, C=64, bf16)",
        "",
        "Made by (from the repository root; OUT is any scratch directory):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "rocprofv3 --kernel-trace --stats -d OUT/stats -o run --output-format csv -- "
        "python3 REPO/bench.py --no-cpu-baseline",
        "rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o run --output-format csv -- "
        f"python3 REPO/bench.py --no-cpu-baseline --steps 5 --warmup 2 --copy-probe-mib {probe_mib}",
        "rocprofv3 --pmc WRITE_SIZE -d OUT/write -o run --output-format csv -- "
        f"python3 REPO/bench.py --no-cpu-baseline --steps 5 --warmup 2 --copy-probe-mib {probe_mib}",
        f"cd REPO && python3 bench.py --summarize OUT/stats OUT/fetch OUT/write {probe_mib}",
        "```",
        "",
        f"Kernel sources hash: `{h}` (bench.py reports traffic only while the sources match).",
        "",
        "## Kernel durations (rocprofv3 --kernel-trace --stats)",
        "",
        "| kernel | calls | mean us | min us | max us |",
        "|---|---|---|---|---|",
    ]
    for r in rows:
        short = _short_kernel(r["Name"])
        if short in KERNELS:
            lines.append(f"| {_kernel_label(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += [
        "",
        "## HBM bytes per launch (FETCH_SIZE, WRITE_SIZE; scaled by a plain copy)",
        "",
        f"A {probe_mib} MiB device-to-device copy in the same runs reads {fkib:.0f} FETCH_SIZE units and "
        f"{wkib:.0f} WRITE_SIZE units: {ffac:.1f} and {wfac:.1f} bytes per unit."
        + ("" if rd is None or wr is None else
           f" Checked on other request mixes of the same size in the same runs: a read-only sum fetches "
           f"{rd:.3f} of its bytes and a write-only fill writes {wr:.3f} of its bytes by these factors."),
        "",
        "| kernel | fetched MB | written MB | total MB |",
        "|---|---|---|---|",
    ]
    for short in ("schedule", "prep", "scan", "decode"):
        ent = traffic.get(KERNELS[short])
        if ent:
            lines.append(f"| {KERNELS[short]} | {ent['fetch_bytes'] / 1e6:.1f} | {ent['write_bytes'] / 1e6:.1f} | "
                         f"{ent['bytes_per_launch'] / 1e6:.1f} |")
    with open(os.path.join(ROOT, "profiles", "gdn_kernels_prefill4096_decode64.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    return traffic, rows


def summarize_short(stats_dir: str, results_jsonl: str):
    """Write profiles/gdn_token_scan_short_prefill.md from a rocprofv3 kernel
    trace of `bench.py --short-prefill` and the JSON lines that run printed."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv"))))
    lines = [
        "# Short prefills: token by token (chunk 1) vs chunked (chunk 64); HK=16, HV=32, d=128, bf16",
        "",
        "Made by (from the repository root; OUT is any scratch directory):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "rocprofv3 --kernel-trace --stats -d OUT/stats -o run --output-format csv -- "
        "python3 REPO/bench.py --short-prefill > OUT/short.jsonl",
        "cd REPO && python3 bench.py --summarize-short OUT/stats OUT/short.jsonl",
        "```",
        "",
        f"Kernel sources hash: `{kernel_source_hash()}`.",
        "",
        "## Kernel durations over all shapes of the run (rocprofv3 --kernel-trace --stats)",
        "",
        "| kernel | calls | mean us | min us | max us |",
        "|---|---|---|---|---|",
    ]
    for r in rows:
        short = _short_kernel(r["Name"])
        if short in KERNELS:
            lines.append(f"| {_kernel_label(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "## Per shape (HIP events in the same run; 4 rotated buffer sets)", "",
              "Taken under the profiler, which adds a per-launch overhead that shows in every column "
              "on the smallest shapes; `python3 bench.py --short-prefill` measures the same without it.", "",
              "| sequences x tokens | token scan us | chunked us | token-scan kernel us | GB/s | chunk 0 picks |",
              "|---|---|---|---|---|---|"]
    for line in open(results_jsonl):
        line = line.strip()
        if not line.startswith("{"):
            continue
        d = json.loads(line)
        lines.append(f"| {d['num_seqs']} x {d['tokens_per_seq']} | {d['token_scan_ms'] * 1e3:.1f} | "
                     f"{d['chunked_ms'] * 1e3:.1f} | {d['token_scan_kernel_ms'] * 1e3:.1f} | "
                     f"{d['token_scan_gbs']:.0f} | {d['chunk0_picks']} |")
    with open(os.path.join(ROOT, "profiles", "gdn_token_scan_short_prefill.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def to_device(x: np.ndarray, dtype: str, dev):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dev)


def device_inputs(inp, dev):
    import torch
    return dict(q=to_device(inp.q, inp.io_dtype, dev), k=to_device(inp.k, inp.io_dtype, dev),
                v=to_device(inp.v, inp.io_dtype, dev), g=to_device(inp.g, inp.gate_dtype, dev),
                beta=to_device(inp.beta, inp.gate_dtype, dev),
                cu_seqlens=torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pre, dec, s_dec, threads: int, one_thread: bool = True):
    """The fp64 oracle on the host cores on the very inputs the GPU step uses:
    the full 4096-token prefill (all 32 value heads) plus one decode step at
    batch 64 from the initial decode states, with `threads` threads and (the
    prefill only, when `one_thread`) with one. Returns the baseline record and
    the oracle's results, which are the bench's parity reference."""
    import oracle
    w = pre.widened()
    t0 = time.perf_counter()
    o_ref, f_ref = oracle.scan(w["q"], w["k"], w["v"], w["g"], w["beta"], w["cu_seqlens"], threads=threads)
    t_pre = time.perf_counter() - t0
    t_pre1 = None
    if one_thread:
        t0 = time.perf_counter()
        oracle.scan(w["q"], w["k"], w["v"], w["g"], w["beta"], w["cu_seqlens"], threads=1)
        t_pre1 = time.perf_counter() - t0
    wd = dec.widened()
    t0 = time.perf_counter()
    od_ref, sd_ref = oracle.decode_step(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"],
                                        s_dec.astype(np.float64), threads=threads)
    t_dec = time.perf_counter() - t0
    rec = {
        "value": (T_PREFILL + B_DECODE) / (t_pre + t_dec), "unit": "tokens/s", "cores": threads,
        "kind": "oracle",
        "sample": f"one full step: prefill T={T_PREFILL} (all {HV} value heads) + decode B={B_DECODE}, "
                  f"fp64 token scan in C; prefill {t_pre:.2f} s, decode {t_dec * 1e3:.1f} ms",
        "prefill_tokens_per_s": T_PREFILL / t_pre,
        "decode_tokens_per_s": B_DECODE / t_dec,
        "prefill_tokens_per_s_one_thread": None if t_pre1 is None else T_PREFILL / t_pre1,
        "cpu_model": _cpu_model(),
        "host_cpus": os.cpu_count(),
    }
    return rec, dict(prefill_out=o_ref, prefill_state=f_ref, decode_out=od_ref, decode_state=sd_ref)


# Parity bars of the bench's gate, as max |gpu - ref| / max |ref| over each
# tensor: bf16 outputs 2e-2; the prefill's final state 2e-2 (bf16 MFMA
# operands in bf16 I/O); the fp32 decode states 1e-4.
PARITY_BARS = {"prefill_out": 2e-2, "prefill_state": 2e-2, "decode_out": 2e-2, "decode_state": 1e-4}


def parity_errors(gpu: dict, ref: dict) -> dict:
    errs = {}
    for key, r in ref.items():
        x = gpu[key]
        den = float(np.abs(r).max())
        diff = np.abs(x - r)
        e = float(diff.max()) / den if den > 0 else float(np.abs(x).max())
        errs[key] = e if np.isfinite(x).all() else float("inf")
    return errs


# Short prefills: (sequences, tokens each). One sequence around the crossover,
# and multi-token steps over a decode-sized batch.
SHORT_SHAPES = ((1, 16), (1, 48), (1, 64), (1, 128), (8, 4), (64, 1), (64, 4), (64, 16))


def short_prefill_sweep(dev, copies, steps):
    """Token-by-token (chunk 1) vs chunked (chunk 64) prefill on short
    prompts and multi-token steps, HK=16, HV=32, d=128, bf16, nonzero initial
    states; one JSON line per shape. The token scan moves the fp32 state
    once in and once out like a decode step, so its rate is also given
    against the HBM peak (algorithmic bytes / kernel time)."""
    import torch
    import gdn_synth as gs
    import gated_deltanet_linear_02_amd as gdn
    for N, k in SHORT_SHAPES:
        T = N * k
        inp = gs.make_inputs([k] * N, HK, HV, D, D, seed=gs.SEED_BASE + 300 + T, io_dtype="bf16",
                             gate_dtype="bf16", init_state=True)
        sets = []
        for _ in range(copies):
            d = device_inputs(inp, dev)
            d["s0"] = torch.from_numpy(inp.initial_state).to(dev)
            d["out"] = torch.empty((T, HV, D), dtype=torch.bfloat16, device=dev)
            d["fin"] = torch.empty((N, HV, D, D), dtype=torch.float32, device=dev)
            d["ws"] = torch.empty(gdn.prefill_workspace_size(N, T, HK, HV, D, D, CHUNK, torch.bfloat16),
                                  dtype=torch.uint8, device=dev)
            sets.append(d)
        res = {}
        for c in (1, CHUNK):
            def run(d):
                gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=c,
                            initial_state=d["s0"], final_state=d["fin"], out=d["out"], workspace=d["ws"])
            for i in range(3):
                run(sets[i % copies])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps):
                run(sets[i % copies])
            e1.record()
            torch.cuda.synchronize()
            res[c] = e0.elapsed_time(e1) / steps
            if c == 1:
                gdn.timing_start(steps)
                for i in range(steps):
                    run(sets[i % copies])
                res["kernel"] = gdn.timing_stop()["token_scan"]["mean_ms"]
        state_bytes = N * HV * D * D * 4 * 2
        io_bytes = T * (2 * HK * D + 2 * HV * D) * 2 + T * HV * 2 * 2
        gbs = (state_bytes + io_bytes) / (res["kernel"] * 1e-3) / 1e9
        auto = {1: "token_scan"}.get(gdn.prefill_method(N, T, HK, HV, D), "chunked")
        print(json.dumps({
            "mode": "short-prefill", "num_seqs": N, "tokens_per_seq": k, "total_tokens": T,
            "token_scan_ms": res[1], "chunked_ms": res[CHUNK], "chunk0_picks": auto,
            "token_scan_speedup": res[CHUNK] / res[1],
            "token_scan_kernel_ms": res["kernel"], "token_scan_gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
            "dtype": "bf16", "data": "synthetic", "buffer_copies": copies,
            "config": {"workload": f"{N} sequence(s) x {k} tokens, HK={HK}, HV={HV}, d={D}"},
        }), flush=True)


def probe_copies(dev, mib):
    """Known-size references for the HBM byte counters of a --pmc run: three
    device-to-device copies of `mib` MiB (they read and write it; the
    counters are scaled by them), and, to check that the same scale holds for
    other request mixes, a fill (writes it only) and three sums (read it only)
    of the same size."""
    if mib <= 0:
        return
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    words = src.view(torch.float32)
    for _ in range(3):
        torch.sum(words)
    torch.cuda.synchronize()
    del src, dst, words


def _probe_check(directory: str, counter: str, factor: float, probe_bytes: int, tag: str):
    """The bytes a probe of probe_bytes moves by `counter` at the copy-derived
    factor, as a fraction of probe_bytes: the largest dispatches (within 10%)
    of torch kernels whose name holds `tag` (FillFunctor: the fill,
    reduce_kernel: the sums). None when the run has no such dispatch."""
    import csv
    vals = []
    with open(os.path.join(directory, "run_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and tag in r["Kernel_Name"] and _short_kernel(r["Kernel_Name"]) == "other":
                vals.append(float(r["Counter_Value"]))
    if not vals:
        return None
    top = max(vals)
    pick = [v for v in vals if v >= 0.9 * top]
    return sum(pick) / len(pick) * factor / probe_bytes


def summarize_norm(stats_dir: str, fetch_dir: str, write_dir: str, results_jsonl: str, probe_mib: int):
    """Write profiles/gdn_output_norm.md from runs of `bench.py --norm`: a
    kernel trace with --stats (whose JSON lines are results_jsonl) and one
    --pmc FETCH_SIZE and one --pmc WRITE_SIZE pass with --copy-probe-mib."""
    import csv
    probe_bytes = probe_mib << 20
    fetch, ffac, fkib = _counter_means(fetch_dir, "FETCH_SIZE", probe_bytes)
    write, wfac, wkib = _counter_means(write_dir, "WRITE_SIZE", probe_bytes)
    rows = list(csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv"))))
    res, pre = {}, []
    for line in open(results_jsonl):
        line = line.strip()
        if line.startswith("{"):
            d = json.loads(line)
            if d["part"] == "prefill":
                pre.append(d)
            else:
                res[d["part"]] = d
    passes = [pp for pp in pre if "algorithmic_bytes" in pp]
    algo = {"decode": decode_bytes_per_step(), "decode_norm": decode_bytes_per_step() + 4 * D,
            "norm_apply": passes[0]["algorithmic_bytes"] if passes else norm_apply_bytes(T_PREFILL)}
    lines = [
        "# Output normalisation: decode batch 64 (fused), prefill 1x4096 and 8x512 in bf16 (fused into the "
        "scan) and 8x512 in fp32 (pass after the scan); HK=16, HV=32, d=128",
        "",
        "Made by (from the repository root; OUT is any scratch directory):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "rocprofv3 --kernel-trace --stats -d OUT/stats -o run --output-format csv -- "
        "python3 REPO/bench.py --norm > OUT/norm.jsonl",
        "rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o run --output-format csv -- "
        f"python3 REPO/bench.py --norm --steps 5 --copy-probe-mib {probe_mib}",
        "rocprofv3 --pmc WRITE_SIZE -d OUT/write -o run --output-format csv -- "
        f"python3 REPO/bench.py --norm --steps 5 --copy-probe-mib {probe_mib}",
        f"cd REPO && python3 bench.py --summarize-norm OUT/stats OUT/fetch OUT/write OUT/norm.jsonl {probe_mib}",
        "```",
        "",
        f"Kernel sources hash: `{kernel_source_hash()}`.",
        "",
        "## Kernel durations (rocprofv3 --kernel-trace --stats)",
        "",
        "The run also launches the plain decode and prefill kernels, for comparison.",
        "",
        "| kernel | calls | mean us | min us | max us |",
        "|---|---|---|---|---|",
    ]
    for r in rows:
        short = _short_kernel(r["Name"])
        if short in KERNELS:
            lines.append(f"| {_kernel_label(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += [
        "",
        "## HBM bytes per launch (FETCH_SIZE, WRITE_SIZE; scaled by a plain copy)",
        "",
        f"A {probe_mib} MiB device-to-device copy in the same runs reads {fkib:.0f} FETCH_SIZE units and "
        f"{wkib:.0f} WRITE_SIZE units: {ffac:.1f} and {wfac:.1f} bytes per unit.",
        "",
        "| kernel | algorithmic MB | fetched MB | written MB | total MB |",
        "|---|---|---|---|---|",
    ]
    for short in ("decode", "decode_norm", "norm_apply"):
        if short in fetch and short in write:
            fb, wb = fetch[short] * ffac, write[short] * wfac
            lines.append(f"| {KERNELS[short]} | {algo[short] / 1e6:.1f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
                         f"{(fb + wb) / 1e6:.1f} |")
    if res or pre:
        dd = res.get("decode")
        lines += ["", "## Rates (HIP events in the traced run)", "",
                  "Taken under the profiler, which adds a per-launch overhead to these event times (compare "
                  "the kernel durations above); `python3 bench.py --norm` measures the same without it.", ""]
        if dd:
            lines.append(f"- decode step, kernel: plain {dd['plain_kernel_ms'] * 1e3:.1f} us, with the norm fused "
                         f"{dd['norm_kernel_ms'] * 1e3:.1f} us ({dd['norm_kernel_gbs']:.0f} GB/s, "
                         f"{100 * dd['hbm_frac']:.1f}% of 8 TB/s).")
        for pp in pre:
            kp = ", ".join(f"{k} {v * 1e3:.1f}" for k, v in pp["plain_kernel_ms"].items())
            kn = ", ".join(f"{k} {v * 1e3:.1f}" for k, v in pp["norm_kernel_ms"].items())
            extra = (f"; the pass at {pp['norm_apply_gbs']:.0f} GB/s, {100 * pp['hbm_frac']:.1f}% of 8 TB/s"
                     if "norm_apply_gbs" in pp else "")
            lines.append(f"- prefill {pp['sequences']}x{pp['tokens'] // pp['sequences']} {pp.get('io', 'bf16')}, "
                         f"{pp.get('rows', '?')}-row slices ({pp['normalisation']}): "
                         f"call plain {pp['plain_ms'] * 1e3:.1f} us, with the norm {pp['norm_ms'] * 1e3:.1f} us; "
                         f"kernel us plain ({kp}), with the norm ({kn}); the norm adds "
                         f"{pp['norm_cost_kernel_us']:.1f} us of kernel time{extra}.")
    with open(os.path.join(ROOT, "profiles", "gdn_output_norm.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_state(stats_dir: str, fetch_dir: str, write_dir: str, results_jsonl: str, probe_mib: int):
    """Write profiles/gdn_decode_state_storage.md from runs of `bench.py
    --bf16-state`: a kernel trace with --stats (whose JSON lines are
    results_jsonl) and one --pmc FETCH_SIZE and one --pmc WRITE_SIZE pass
    with --copy-probe-mib."""
    import csv
    probe_bytes = probe_mib << 20
    fetch, ffac, fkib = _counter_means(fetch_dir, "FETCH_SIZE", probe_bytes, key=_state_key)
    write, wfac, wkib = _counter_means(write_dir, "WRITE_SIZE", probe_bytes, key=_state_key)
    rows = list(csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv"))))
    lines = [
        f"# Decode batch {B_DECODE} with fp32 and bf16 state storage (HK={HK}, HV={HV}, d={D}, bf16 I/O)",
        "",
        "Made by (from the repository root; OUT is any scratch directory):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "rocprofv3 --kernel-trace --stats -d OUT/stats -o run --output-format csv -- "
        "python3 REPO/bench.py --bf16-state > OUT/state.jsonl",
        "rocprofv3 --pmc FETCH_SIZE -d OUT/fetch -o run --output-format csv -- "
        f"python3 REPO/bench.py --bf16-state --steps 5 --copy-probe-mib {probe_mib}",
        "rocprofv3 --pmc WRITE_SIZE -d OUT/write -o run --output-format csv -- "
        f"python3 REPO/bench.py --bf16-state --steps 5 --copy-probe-mib {probe_mib}",
        f"cd REPO && python3 bench.py --summarize-state OUT/stats OUT/fetch OUT/write OUT/state.jsonl {probe_mib}",
        "```",
        "",
        f"Kernel sources hash: `{kernel_source_hash()}`.",
        "",
        "## Kernel durations (rocprofv3 --kernel-trace --stats)",
        "",
        "| kernel | state | calls | mean us | min us | max us |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows:
        k = _state_key(r["Name"])
        short = k.split("/")[0]
        if short in ("decode", "decode_norm"):
            lines.append(f"| {_kernel_label(r['Name'])} | {'bf16' if k.endswith('/bf16') else 'fp32'} | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} |")
    lines += [
        "",
        "## HBM bytes per launch (FETCH_SIZE, WRITE_SIZE; scaled by a plain copy)",
        "",
        f"A {probe_mib} MiB device-to-device copy in the same runs reads {fkib:.0f} FETCH_SIZE units and "
        f"{wkib:.0f} WRITE_SIZE units: {ffac:.1f} and {wfac:.1f} bytes per unit.",
        "",
        "| kernel | state | algorithmic MB | fetched MB | written MB | total MB |",
        "|---|---|---|---|---|---|",
    ]
    for k in ("decode", "decode/bf16", "decode_norm", "decode_norm/bf16"):
        if k in fetch and k in write:
            short, bf = k.split("/")[0], k.endswith("/bf16")
            algo = decode_bytes_per_step(state_bytes=2 if bf else 4) + (4 * D if short == "decode_norm" else 0)
            fb, wb = fetch[k] * ffac, write[k] * wfac
            lines.append(f"| {KERNELS[short]} | {'bf16' if bf else 'fp32'} | {algo / 1e6:.1f} | {fb / 1e6:.1f} | "
                         f"{wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} |")
    lines += ["", "## Rates (HIP events in the traced run)", "",
              "Taken under the profiler, which adds a per-launch overhead to these event times; "
              "`python3 bench.py --bf16-state` measures the same without it.", "",
              "| state | norm | kernel us | tokens/s | GB/s | of 8 TB/s |", "|---|---|---|---|---|---|"]
    for line in open(results_jsonl):
        line = line.strip()
        if line.startswith("{"):
            d = json.loads(line)
            lines.append(f"| {d['state_dtype']} | {'fused' if d['norm'] else 'no'} | {d['kernel_ms'] * 1e3:.1f} | "
                         f"{d['tokens_per_s'] / 1e6:.2f} M | {d['kernel_gbs']:.0f} | {100 * d['hbm_frac']:.1f}% |")
    with open(os.path.join(ROOT, "profiles", "gdn_decode_state_storage.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def _lengths_label(lens) -> str:
    """Sequence lengths with runs grouped: 4096 + 4 x 512."""
    parts, i = [], 0
    while i < len(lens):
        j = i
        while j < len(lens) and lens[j] == lens[i]:
            j += 1
        parts.append(str(lens[i]) if j - i == 1 else f"{j - i} x {lens[i]}")
        i = j
    return " + ".join(parts)


def summarize_tune(stats_dir: str, results_jsonl: str):
    """Write profiles/gdn_prefill_tuning.md from a rocprofv3 kernel trace of
    `bench.py --tune` (kernel durations) and the JSON lines of a second
    `bench.py --tune` run made without the profiler (the per-shape timings:
    the profiler's per-launch overhead distorts the short launches these
    shapes compare)."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv"))))
    lines = [
        f"# Prefill method chosen by measurement vs the fixed rule; HK={HK}, HV={HV}, d={D}, bf16",
        "",
        "Made by (from the repository root; OUT is any scratch directory):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "rocprofv3 --kernel-trace --stats -d OUT/stats -o run --output-format csv -- "
        "python3 REPO/bench.py --tune > OUT/tune_profiled.jsonl",
        "python3 REPO/bench.py --tune > OUT/tune.jsonl",
        "cd REPO && python3 bench.py --summarize-tune OUT/stats OUT/tune.jsonl",
        "```",
        "",
        f"Kernel sources hash: `{kernel_source_hash()}`.",
        "",
        "## Kernel durations over the whole run (rocprofv3 --kernel-trace --stats)",
        "",
        "| kernel | calls | mean us | min us | max us |",
        "|---|---|---|---|---|",
    ]
    import re
    for r in rows:
        short = _short_kernel(r["Name"])
        if short in KERNELS or "gate_kernel" in r["Name"]:
            name = _kernel_label(r["Name"]) if short in KERNELS else "gdn_gate_kernel"
            if "gate_kernel" in r["Name"]:
                name += " (bf16)" if ("IDF16b" in r["Name"] or "_Accum" in r["Name"]) else " (fp32)"
            lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "## Per shape (HIP events, run without the profiler)", "",
              "chunk 0 timed on rotated buffer sets under the fixed rule (empty cache; the better of a run "
              "before and one after) and under the tuned choice; the candidates' own times are the tuner's "
              "(warm, same inputs). The rule agrees with the tuner when it picks the tuner's fastest "
              "candidate or one within 5% of it (last column).", "",
              "Methods are named chunk/rows: chunk size, then state rows per scan workgroup; 1 is token by "
              "token.", "",
              "| sequences x tokens | rule | rule us | tuned | tuned us | speedup | tuner's warm us per method "
              "| rule's candidate / fastest |",
              "|---|---|---|---|---|---|---|---|"]
    results = [json.loads(x) for x in (y.strip() for y in open(results_jsonl)) if x.startswith("{")]
    for d in results:
        if d.get("lengths"):
            continue
        cand = d["candidate_ms_warm"]
        warm = ", ".join(f"{c}: {t * 1e3:.1f}" if t >= 0 else f"{c}: -" for c, t in cand.items())
        best = min(t for t in cand.values() if t >= 0)
        ratio = cand.get(d["rule_method"], -1) / best if cand.get(d["rule_method"], -1) > 0 else float("nan")
        lines.append(f"| {d['num_seqs']} x {d['tokens_per_seq']} | {d['rule_method']} | {d['rule_ms'] * 1e3:.1f} | "
                     f"{d['tuned_method']} | {d['tuned_ms'] * 1e3:.1f} | {d['speedup']:.2f} | {warm} | "
                     f"{ratio:.2f} |")
    uneven = [d for d in results if d.get("lengths")]
    if uneven:
        lines += ["", "## Uneven batches: the rule with and without the max_seqlen hint", "",
                  "The same protocol, on batches of unequal sequences. The hinted method is the rule's choice "
                  "when the caller passes the longest length (gdn_prefill_hint); without it the rule sees only "
                  "the sizes.", "",
                  "| lengths | rule | rule us | hinted | hinted us | rule / hinted | tuned | tuned us | "
                  "hinted's candidate / fastest |",
                  "|---|---|---|---|---|---|---|---|---|"]
        for d in uneven:
            cand = d["candidate_ms_warm"]
            best = min(t for t in cand.values() if t >= 0)
            hc = cand.get(d["hinted_method"], -1)
            ratio = hc / best if hc > 0 else float("nan")
            lines.append(f"| {_lengths_label(d['lengths'])} | {d['rule_method']} | {d['rule_ms'] * 1e3:.1f} | "
                         f"{d['hinted_method']} | {d['hinted_ms'] * 1e3:.1f} | {d['rule_ms'] / d['hinted_ms']:.2f} | "
                         f"{d['tuned_method']} | {d['tuned_ms'] * 1e3:.1f} | {ratio:.2f} |")
    with open(os.path.join(ROOT, "profiles", "gdn_prefill_tuning.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_mfma(pmc_dir: str, stats_dir: str):
    """Write profiles/gdn_mfma_counters.md: MFMA work counted by the hardware
    (SQ_INSTS_VALU_MFMA_MOPS_*, 512 flops per unit) per launch of the
    preparation and scan kernels, beside their algorithmic flops, and the
    rates both give over the kernels' mean durations (kernel trace)."""
    import csv
    per = {}
    for r in csv.DictReader(open(os.path.join(pmc_dir, "run_counter_collection.csv"))):
        short = _short_kernel(r["Kernel_Name"])
        if short in ("prep", "scan"):
            per.setdefault(short, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    dur = {}
    for r in csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv"))):
        short = _short_kernel(r["Name"])
        if short in ("prep", "scan"):
            dur[short] = float(r["AverageNs"]) * 1e-9
    algo = {"scan": scan_flops_per_token() * T_PREFILL, "prep": prep_flops_per_token() * T_PREFILL}
    lines = [
        f"# MFMA work counted by the hardware: prefill 1x{T_PREFILL} (HK={HK}, HV={HV}, d={D}, C={CHUNK}, bf16)",
        "",
        "Made by (from the repository root; OUT is any scratch directory):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 SQ_VALU_MFMA_BUSY_CYCLES "
        "SQ_BUSY_CYCLES GRBM_GUI_ACTIVE -d OUT/mfma -o run --output-format csv -- "
        "python3 REPO/bench.py --no-cpu-baseline --steps 5 --warmup 2",
        "rocprofv3 --kernel-trace --stats -d OUT/stats -o run --output-format csv -- "
        "python3 REPO/bench.py --no-cpu-baseline --steps 20",
        "cd REPO && python3 bench.py --summarize-mfma OUT/mfma OUT/stats",
        "```",
        "",
        f"Kernel sources hash: `{kernel_source_hash()}`. One MOPS unit is 512 flops.",
        "",
        "| kernel | counted bf16 GFLOP | counted fp32 GFLOP | algorithmic GFLOP | counted / algorithmic "
        "| mean us | counted TFLOP/s | algorithmic TFLOP/s | of 2.5 PFLOP/s bf16 (counted) |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    for k in ("prep", "scan"):
        c = per.get(k, {})
        if not c or k not in dur:
            continue
        bf = sum(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0])) / max(1, len(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0]))) * 512
        f32 = sum(c.get("SQ_INSTS_VALU_MFMA_MOPS_F32", [0])) / max(1, len(c.get("SQ_INSTS_VALU_MFMA_MOPS_F32", [0]))) * 512
        t = dur[k]
        lines.append(f"| {KERNELS[k]} | {bf / 1e9:.2f} | {f32 / 1e9:.3f} | {algo[k] / 1e9:.2f} | {bf / algo[k]:.2f} | "
                     f"{t * 1e6:.1f} | {bf / t / 1e12:.0f} | {algo[k] / t / 1e12:.0f} | "
                     f"{100 * bf / t / 1e12 / PEAK_BF16_TFLOPS:.1f}% |")
    lines += ["", "Counted below algorithmic: the kernels skip the zero blocks of the triangular T and P "
              "(the algorithmic count takes full C x C tiles); the preparation kernel's fp32 MFMA is the "
              "blocked triangular inverse. Raw means per launch (sums over the device's XCDs, SEs or SIMDs "
              "as each counter defines):", ""]
    for k in ("prep", "scan"):
        if k in per:
            lines.append(f"- {KERNELS[k]}: " + ", ".join(f"{n} {sum(v) / len(v):.0f}" for n, v in sorted(per[k].items())))
    with open(os.path.join(ROOT, "profiles", "gdn_mfma_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_configs(stats_dir: str, results_jsonl: str):
    """Write profiles/gdn_long_varlen.md from a rocprofv3 kernel trace of
    `bench.py --configs` and the JSON lines that run printed."""
    import csv
    import re
    rows = list(csv.DictReader(open(os.path.join(stats_dir, "run_kernel_stats.csv"))))
    lines = [
        f"# Long (T = 32768) and varlen (8 sequences, then 64 decode steps at batch 8) workloads; "
        f"HK={HK}, HV={HV}, d={D}, bf16",
        "",
        "Made by (from the repository root; OUT is any scratch directory):",
        "",
        "```",
        "cd /tmp && export TMPDIR=/tmp",
        "rocprofv3 --kernel-trace --stats -d OUT/stats -o run --output-format csv -- "
        "python3 REPO/bench.py --configs > OUT/configs.jsonl",
        "cd REPO && python3 bench.py --summarize-configs OUT/stats OUT/configs.jsonl",
        "```",
        "",
        f"Kernel sources hash: `{kernel_source_hash()}`.",
        "",
        "## Kernel durations over the run (rocprofv3 --kernel-trace --stats)",
        "",
        "Both prefills' launches are averaged together; the per-workload kernel means follow below.",
        "",
        "| kernel | calls | mean us | min us | max us |",
        "|---|---|---|---|---|",
    ]
    for r in rows:
        short = _short_kernel(r["Name"])
        if short in KERNELS:
            lines.append(f"| {_kernel_label(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "## Per workload (HIP events in the same run, under the profiler)", "",
              "Methods are named chunk/rows (chunk size, state rows per scan workgroup). The first is chunk "
              "64 with the rule's rows, which the kernel columns describe. The hinted method is the rule's "
              "choice when the caller passes the longest length (max_seqlen, gdn_prefill_hint); the tuned "
              "method is the one gdn_tune_prefill picks for the workload (the host-side rule sees sizes, "
              "not the lengths). The decode step at batch 8 is timed two ways: back-to-back eager launches "
              "from Python (bound by the host at this size) and the kernel's own events; under the profiler "
              "both read several times longer than without it (kernel about 6.4 us, eager step about "
              "12 us in a plain run of `bench.py --configs`).", "",
              "| workload | sequences | tokens | method | prefill ms | tokens/s | prep ms | scan ms | scan MFMA | "
              "hinted method | hinted prefill ms | tuned method | tuned prefill ms | tuned tokens/s | "
              "decode b8 step us: eager / kernel |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for line in open(results_jsonl):
        line = line.strip()
        if not line.startswith("{"):
            continue
        d = json.loads(line)
        km = d["kernel_ms"]
        dec = (f"{d['decode_b8_step_ms'] * 1e3:.1f} / {d['decode_b8_kernel_ms'] * 1e3:.1f}"
               if "decode_b8_step_ms" in d else "-")
        lines.append(f"| {d['workload']} | {d['num_seqs']} | {d['total_tokens']} | {d['method']} | "
                     f"{d['prefill_ms']:.3f} | {d['tokens_per_s'] / 1e6:.1f} M | {km['prep']:.3f} | "
                     f"{km['scan']:.3f} | {100 * d['scan_mfma_frac']:.1f}% | {d['hinted_method']} | "
                     f"{d['hinted_prefill_ms']:.3f} | {d['tuned_method']} | "
                     f"{d['tuned_prefill_ms']:.3f} | {d['tuned_tokens_per_s'] / 1e6:.1f} M | {dec} |")
    with open(os.path.join(ROOT, "profiles", "gdn_long_varlen.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def norm_apply_bytes(tokens, hv=HV, dv=D, elem=2):
    """Algorithmic HBM bytes of the prefill's output-normalisation pass: every
    output row read and written once (the weight and cu_seqlens are a few
    hundred bytes)."""
    return 2 * tokens * hv * dv * elem


def output_norm_bench(dev, copies, steps):
    """Output normalisation: decode B=64 with the fused kernel against the
    plain one, and three prefills against the plain prefill: one 4096-token
    sequence (16-row scan slices, which exchange partial sums: the
    normalisation fused into the scan), eight 512-token sequences (128-row
    slices, each a whole head: fused, no exchange), and the same eight in
    fp32 I/O (16-row slices over several passes: a pass after the scan).
    One JSON line each; kernel times from the library's dispatch-stamped
    events."""
    import torch
    import gdn_synth as gs
    import gated_deltanet_linear_02_amd as gdn
    w = torch.from_numpy(gs.norm_weight(D, seed=gs.SEED_BASE + 505)).to(dev)
    eps = 1e-6

    def measure(run, sets, kinds):
        for i in range(3):
            run(sets[i % copies])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            run(sets[i % copies])
        e1.record()
        torch.cuda.synchronize()
        call_ms = e0.elapsed_time(e1) / steps
        gdn.timing_start(8 * steps)
        for i in range(steps):
            run(sets[i % copies])
        kt = gdn.timing_stop()
        return call_ms, {k: kt[k]["mean_ms"] for k in kinds}

    dec = gs.workload("decode", batch=B_DECODE)
    s_dec = gs.decode_state(B_DECODE, HV, D, D, seed=gs.SEED_BASE + 101)
    dsets = []
    for _ in range(copies):
        d = device_inputs(dec, dev)
        d["state"] = torch.from_numpy(s_dec).to(dev)
        d["out"] = torch.empty((B_DECODE, HV, D), dtype=torch.bfloat16, device=dev)
        dsets.append(d)
    plain_ms, plain_k = measure(lambda d: gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                                          out=d["out"]), dsets, ("decode",))
    norm_ms, norm_k = measure(lambda d: gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                                        out=d["out"], norm_weight=w, norm_eps=eps),
                              dsets, ("decode_norm",))
    by = decode_bytes_per_step() + 4 * D
    gbs = by / (norm_k["decode_norm"] * 1e-3) / 1e9
    print(json.dumps({
        "mode": "output-norm", "part": "decode", "plain_ms": plain_ms, "norm_ms": norm_ms,
        "plain_kernel_ms": plain_k["decode"], "norm_kernel_ms": norm_k["decode_norm"],
        "norm_kernel_gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes": by,
        "dtype": "bf16", "data": "synthetic", "buffer_copies": copies,
        "config": {"workload": f"decode batch {B_DECODE}, HK={HK}, HV={HV}, d={D}, fp32 state; "
                               f"RMS output norm, eps {eps}"},
    }), flush=True)
    del dsets

    # prefill: the headline shape and eight sequences, bf16 (the
    # normalisation fused into the scan), and eight in fp32 (a pass after it)
    for lens, io in (([T_PREFILL], "bf16"), ([512] * 8, "bf16"), ([512] * 8, "f32")):
        n, tt = len(lens), sum(lens)
        io_dt = torch.bfloat16 if io == "bf16" else torch.float32
        pre = gs.make_inputs(lens, HK, HV, D, D, seed=gs.SEED_BASE + 2, io_dtype=io, gate_dtype="f32") \
            if n > 1 else gs.workload("prefill")
        ws_bytes = gdn.prefill_workspace_size(n, tt, HK, HV, D, D, CHUNK, io_dt)
        rows = gdn.prefill_plan(n, tt, HK, HV, D, CHUNK, io_dt)[1]
        psets = []
        for _ in range(copies):
            d = device_inputs(pre, dev)
            d["out"] = torch.empty((tt, HV, D), dtype=io_dt, device=dev)
            d["fin"] = torch.empty((n, HV, D, D), dtype=torch.float32, device=dev)
            d["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            psets.append(d)

        def pre_run(d, norm):
            gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=CHUNK,
                        final_state=d["fin"], out=d["out"], workspace=d["ws"],
                        norm_weight=w if norm else None, norm_eps=eps)
        kinds = ("schedule", "prep", "scan", "norm_apply")
        plain_ms, pk = measure(lambda d: pre_run(d, False), psets, kinds)
        norm_ms, nk = measure(lambda d: pre_run(d, True), psets, kinds)
        fused = nk["norm_apply"] == 0.0
        rec = {
            "mode": "output-norm", "part": "prefill", "sequences": n, "tokens": tt, "io": io, "rows": rows,
            "normalisation": ("fused into the scan" + (" (whole-head slices)" if rows == D else
                                                        " (exchange between slices)")) if fused
            else "pass after the scan",
            "plain_ms": plain_ms, "norm_ms": norm_ms,
            "plain_kernel_ms": {k: pk[k] for k in kinds if pk[k] > 0},
            "norm_kernel_ms": {k: nk[k] for k in kinds if nk[k] > 0},
            "norm_cost_kernel_us": 1e3 * (sum(nk.values()) - sum(pk.values())),
            "dtype": io, "data": "synthetic", "buffer_copies": copies,
            "config": {"workload": f"prefill {n}x{tt // n} tokens, HK={HK}, HV={HV}, d={D}, chunk {CHUNK}, "
                                   f"{rows}-row scan slices; RMS output norm, eps {eps}"},
        }
        if not fused:
            by = norm_apply_bytes(tt, elem=4 if io == "f32" else 2)
            gbs = by / (nk["norm_apply"] * 1e-3) / 1e9
            rec.update({"norm_apply_gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes": by})
        print(json.dumps(rec), flush=True)
        del psets


def state_storage_bench(dev, copies, steps):
    """Decode batch 64 with the state pool stored in fp32 and in bf16 (fp32
    arithmetic either way), without and with the fused output norm. One JSON
    line per case; kernel times from the library's dispatch-stamped events,
    HBM rate from the algorithmic bytes (state read and written once, plus
    q, k, v, gates and output)."""
    import torch
    import gdn_synth as gs
    import gated_deltanet_linear_02_amd as gdn
    w = torch.from_numpy(gs.norm_weight(D, seed=gs.SEED_BASE + 505)).to(dev)
    dec = gs.workload("decode", batch=B_DECODE)
    s_dec = gs.decode_state(B_DECODE, HV, D, D, seed=gs.SEED_BASE + 101)
    for sdt in (torch.float32, torch.bfloat16):
        sets = []
        for _ in range(copies):
            d = device_inputs(dec, dev)
            d["state"] = torch.from_numpy(s_dec).to(dev).to(sdt)
            d["out"] = torch.empty((B_DECODE, HV, D), dtype=torch.bfloat16, device=dev)
            sets.append(d)
        for norm in (False, True):
            def run(d):
                gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], out=d["out"],
                                norm_weight=w if norm else None)
            for i in range(3):
                run(sets[i % copies])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps):
                run(sets[i % copies])
            e1.record()
            torch.cuda.synchronize()
            call_ms = e0.elapsed_time(e1) / steps
            gdn.timing_start(steps)
            for i in range(steps):
                run(sets[i % copies])
            kind = "decode_norm" if norm else "decode"
            kms = gdn.timing_stop()[kind]["mean_ms"]
            sb = 2 if sdt == torch.bfloat16 else 4
            by = decode_bytes_per_step(state_bytes=sb) + (4 * D if norm else 0)
            gbs = by / (kms * 1e-3) / 1e9
            print(json.dumps({
                "mode": "state-storage", "state_dtype": "bf16" if sb == 2 else "f32", "norm": norm,
                "call_ms": call_ms, "kernel_ms": kms, "tokens_per_s": B_DECODE / (kms * 1e-3),
                "kernel_gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes": by,
                "dtype": "bf16", "data": "synthetic", "buffer_copies": copies,
                "config": {"workload": f"decode batch {B_DECODE}, HK={HK}, HV={HV}, d={D}"},
            }), flush=True)


def configs_bench(dev, reps):
    """The long and varlen workloads, timed (they are parity cases in the
    tests; here only their speed): a 32768-token prefill from an initial
    state, and 8 packed sequences of 256 to 16384 tokens followed by 64
    decode steps at batch 8 from their final states. HK=16, HV=32, d=128,
    bf16 I/O, fp32 gates and states, chunk 64 with the state rows per scan
    workgroup of the rule; the rule given the longest length as a hint
    (max_seqlen, chunk 0); then the method gdn_tune_prefill picks for the
    workload (chunk 0 after tuning). One JSON line each."""
    import torch
    import gdn_synth as gs
    import gated_deltanet_linear_02_amd as gdn

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for name in ("long", "varlen"):
        inp = gs.workload(name)
        d = device_inputs(inp, dev)
        N, T = inp.num_seqs, inp.total_tokens
        s0 = torch.from_numpy(inp.initial_state).to(dev)
        fin = torch.empty_like(s0)
        out = torch.empty((T, HV, D), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(gdn.prefill_workspace_size(N, T, HK, HV, D, D, 0, torch.bfloat16),
                         dtype=torch.uint8, device=dev)
        lmax = int(np.diff(inp.cu_seqlens).max())

        def run(chunk=CHUNK, hint=None):
            gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=chunk,
                        initial_state=s0, final_state=fin, out=out, workspace=ws, max_seqlen=hint)

        gdn.tune_cache_clear()
        method = gdn.method_name(*gdn.prefill_plan(N, T, HK, HV, D, CHUNK))
        ms = timed(run, reps)
        gdn.timing_start(8 * reps)
        for _ in range(reps):
            run()
        kt = gdn.timing_stop()
        scan_ms = kt["scan"]["mean_ms"]
        hinted = gdn.method_name(*gdn.prefill_plan(N, T, HK, HV, D, 0, max_seqlen=lmax))
        hinted_ms = timed(lambda: run(0, lmax), reps)
        tuned = gdn.tune_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], initial_state=s0)
        tuned_ms = timed(lambda: run(0), reps)
        gdn.tune_cache_clear()
        ms = min(ms, timed(run, reps))  # the rule's method before and after, so that order favours neither
        res = {"mode": "configs", "workload": name, "num_seqs": N, "total_tokens": T, "method": method,
               "prefill_ms": ms, "tokens_per_s": T / (ms * 1e-3),
               "kernel_ms": {k: kt[k]["mean_ms"] for k in ("schedule", "prep", "scan")},
               "scan_mfma_frac": scan_flops_per_token() * T / (scan_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               "hinted_method": hinted, "hinted_prefill_ms": hinted_ms, "max_seqlen": lmax,
               "tuned_method": tuned["method"], "tuned_prefill_ms": tuned_ms,
               "tuned_tokens_per_s": T / (tuned_ms * 1e-3),
               "dtype": "bf16", "data": "synthetic",
               "config": {"workload": f"{name}: {N} sequence(s), {T} tokens, HK={HK}, HV={HV}, d={D}, chunk {CHUNK}",
                          "lengths": np.diff(inp.cu_seqlens).tolist()}}
        if name == "varlen":
            # 64 decode steps at batch 8 continuing from the final states
            dec = device_inputs(gs.make_inputs([1] * N, HK, HV, D, D, seed=gs.SEED_BASE + 404, io_dtype="bf16",
                                               gate_dtype="bf16"), dev)
            state = fin.clone()
            dout = torch.empty((N, HV, D), dtype=torch.bfloat16, device=dev)

            def dstep():
                gdn.decode_step(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], state, out=dout)

            # eager launches from Python (bound by the host at this size) and
            # the kernel's own time
            step_ms = timed(dstep, 64)
            gdn.timing_start(64)
            for _ in range(64):
                dstep()
            dk = gdn.timing_stop()
            res["decode_b8_step_ms"] = step_ms
            res["decode_b8_kernel_ms"] = dk["decode"]["mean_ms"]
            res["decode_b8_tokens_per_s"] = N / (step_ms * 1e-3)
        print(json.dumps(res), flush=True)
        del d, out, ws, s0, fin
        torch.cuda.empty_cache()


def graph_bench(dev, steps):
    """One decode step per token, launched eagerly (Python, ctypes, one HIP
    launch) against the same step captured once in a HIP graph and replayed,
    at batch 1, 8 and 64 (HK=16, HV=32, d=128, bf16, fp32 states). One JSON
    line per batch; times from events around `steps` back-to-back steps."""
    import torch
    import gdn_synth as gs
    import gated_deltanet_linear_02_amd as gdn
    for B in (1, 8, 64):
        d = device_inputs(gs.make_inputs([1] * B, HK, HV, D, D, seed=gs.SEED_BASE + 1, io_dtype="bf16",
                                         gate_dtype="bf16"), dev)
        state = torch.from_numpy(gs.decode_state(B, HV, D, D, seed=gs.SEED_BASE + 101)).to(dev)
        out = torch.empty((B, HV, D), dtype=torch.bfloat16, device=dev)

        def step():
            gdn.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], state, out=out)

        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()

        def timed(fn):
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps

        eager_ms, graph_ms = timed(step), timed(graph.replay)
        gdn.timing_start(steps)
        for _ in range(steps):
            step()
        kms = gdn.timing_stop()["decode"]["mean_ms"]
        print(json.dumps({
            "mode": "graph", "batch": B, "eager_ms": eager_ms, "graph_ms": graph_ms, "kernel_ms": kms,
            "eager_tokens_per_s": B / (eager_ms * 1e-3), "graph_tokens_per_s": B / (graph_ms * 1e-3),
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"decode batch {B}, HK={HK}, HV={HV}, d={D}, fp32 state"},
        }), flush=True)


# Shapes for the tuning sweep: (sequences, tokens each).
TUNE_SHAPES = ((1, 16), (1, 48), (1, 128), (1, 512), (8, 4), (64, 1), (64, 4), (64, 16), (16, 16), (32, 24),
               (32, 128), (8, 300), (2, 600), (8, 512), (4, 1024), (2, 2048), (1, 4096))
# Uneven batches (token counts per sequence), where the rule's choice also
# depends on the longest length when the caller gives it (max_seqlen).
UNEVEN_SHAPES = ((4096, 512, 512, 512, 512), (8192, 1024, 1024), (2048, 2048, 128, 128, 128, 128),
                 (3000,) + (100,) * 10, (6000, 3000, 1500, 750), (2048, 1024, 512, 256), (300, 77, 5),
                 (1000, 100, 100, 100), (500,) + (1,) * 63, (120,) + (3,) * 20)


def tuning_sweep(dev, copies, steps):
    """gdn_tune_prefill on each shape, then prefill with chunk 0 timed under
    the fixed rule (empty cache) and under the tuned choice, on rotated buffer
    sets (cold caches); uneven batches also under the rule given the longest
    length (max_seqlen). HK=16, HV=32, d=128, bf16, fp32 gates, nonzero
    initial states; one JSON line per shape."""
    import torch
    import gdn_synth as gs
    import gated_deltanet_linear_02_amd as gdn
    shapes = [[k] * N for N, k in TUNE_SHAPES] + [list(u) for u in UNEVEN_SHAPES]
    for lens in shapes:
        N, T, k = len(lens), sum(lens), lens[0]
        uneven = len(set(lens)) > 1
        inp = gs.make_inputs(lens, HK, HV, D, D, seed=gs.SEED_BASE + 900 + T + (N if uneven else 0),
                             io_dtype="bf16", gate_dtype="f32", init_state=True)
        sets = []
        for _ in range(copies):
            d = device_inputs(inp, dev)
            d["s0"] = torch.from_numpy(inp.initial_state).to(dev)
            d["out"] = torch.empty((T, HV, D), dtype=torch.bfloat16, device=dev)
            d["fin"] = torch.empty((N, HV, D, D), dtype=torch.float32, device=dev)
            d["ws"] = torch.empty(gdn.prefill_workspace_size(N, T, HK, HV, D, D, 0, torch.bfloat16),
                                  dtype=torch.uint8, device=dev)
            sets.append(d)

        def run(d, hint=None):
            gdn.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], chunk=0,
                        initial_state=d["s0"], final_state=d["fin"], out=d["out"], workspace=d["ws"],
                        max_seqlen=hint)

        def timed(hint=None):
            for i in range(3):
                run(sets[i % copies], hint)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps):
                run(sets[i % copies], hint)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps

        # the rule is timed before and after the tuned choice (the better of
        # the two counts), so that warm-up order favours neither
        gdn.tune_cache_clear()
        rule_ms = timed()
        rule = gdn.method_name(*gdn.prefill_plan(N, T, HK, HV, D))
        hinted = gdn.method_name(*gdn.prefill_plan(N, T, HK, HV, D, max_seqlen=max(lens)))
        hinted_ms = timed(max(lens)) if uneven else rule_ms
        d0 = sets[0]
        r = gdn.tune_prefill(d0["q"], d0["k"], d0["v"], d0["g"], d0["beta"], d0["cu_seqlens"], initial_state=d0["s0"])
        tuned_ms = timed()
        gdn.tune_cache_clear()
        rule_ms = min(rule_ms, timed())
        if not uneven:
            hinted_ms = rule_ms
        print(json.dumps({
            "mode": "tuning", "num_seqs": N, "tokens_per_seq": k, "total_tokens": T,
            "lengths": lens if uneven else None, "hinted_method": hinted, "hinted_ms": hinted_ms,
            "rule_method": rule, "tuned_method": r["method"], "rule_ms": rule_ms, "tuned_ms": tuned_ms,
            "speedup": rule_ms / tuned_ms, "candidate_ms_warm": r["ms"], "candidate_gate_err": r["err"],
            "dtype": "bf16", "data": "synthetic", "buffer_copies": copies,
            "config": {"workload": (f"{N} sequences of {'+'.join(map(str, lens))} tokens" if uneven
                                    else f"{N} sequence(s) x {k} tokens") + f", HK={HK}, HV={HV}, d={D}"},
        }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="buffer sets rotated through (cold caches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--short-prefill", action="store_true",
                    help="instead of the main line: token-by-token vs chunked prefill on short prompts "
                         "and multi-token steps, one JSON line per shape")
    ap.add_argument("--norm", action="store_true",
                    help="instead of the main line: decode and prefill with the output normalisation "
                         "against the plain calls, one JSON line each")
    ap.add_argument("--bf16-state", action="store_true",
                    help="instead of the main line: decode with fp32 and with bf16 state storage, "
                         "one JSON line per case")
    ap.add_argument("--tune", action="store_true",
                    help="instead of the main line: tune the prefill method per shape and time chunk 0 "
                         "under the fixed rule and under the tuned choice, one JSON line per shape")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the main line: time the long (T=32768) and varlen (8 sequences + 64 "
                         "decode steps) workloads, one JSON line each")
    ap.add_argument("--graph", action="store_true",
                    help="instead of the main line: decode steps launched eagerly vs replayed from a HIP graph")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before warm-up, run 3 device-to-device copies of this many MiB "
                         "(the known-size reference for HBM byte counters)")
    ap.add_argument("--summarize", nargs=4, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR", "PROBE_MIB"),
                    help="host only: turn rocprofv3 output directories into the summaries under "
                         "profiles/ and exit")
    ap.add_argument("--summarize-short", nargs=2, metavar=("STATS_DIR", "RESULTS_JSONL"),
                    help="host only: turn a kernel trace of --short-prefill into "
                         "profiles/gdn_token_scan_short_prefill.md and exit")
    ap.add_argument("--summarize-norm", nargs=5,
                    metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR", "RESULTS_JSONL", "PROBE_MIB"),
                    help="host only: turn rocprofv3 runs of --norm into profiles/gdn_output_norm.md and exit")
    ap.add_argument("--summarize-state", nargs=5,
                    metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR", "RESULTS_JSONL", "PROBE_MIB"),
                    help="host only: turn rocprofv3 runs of --bf16-state into "
                         "profiles/gdn_decode_state_storage.md and exit")
    ap.add_argument("--summarize-tune", nargs=2, metavar=("STATS_DIR", "RESULTS_JSONL"),
                    help="host only: turn a kernel trace of --tune into profiles/gdn_prefill_tuning.md and exit")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "STATS_DIR"),
                    help="host only: turn an MFMA counter run and a kernel trace into "
                         "profiles/gdn_mfma_counters.md and exit")
    ap.add_argument("--summarize-configs", nargs=2, metavar=("STATS_DIR", "RESULTS_JSONL"),
                    help="host only: turn a kernel trace of --configs into profiles/gdn_long_varlen.md and exit")
    args = ap.parse_args()

    if args.summarize_configs:
        summarize_configs(*args.summarize_configs)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.summarize_tune:
        summarize_tune(*args.summarize_tune)
        return
    if args.summarize_state:
        summarize_state(*args.summarize_state[:4], int(args.summarize_state[4]))
        return
    if args.summarize_norm:
        summarize_norm(*args.summarize_norm[:4], int(args.summarize_norm[4]))
        return
    if args.summarize:
        summarize_profiles(*args.summarize[:3], int(args.summarize[3]))
        return
    if args.summarize_short:
        summarize_short(*args.summarize_short)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this layer's path is built and measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)

    import torch
    import gdn_synth as gs
    import gated_deltanet_linear_02_amd as gdn

    if torch.cuda.device_count() < 1:
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.short_prefill:
        short_prefill_sweep(dev, args.copies, min(args.steps, 30))
        return
    if args.tune:
        tuning_sweep(dev, args.copies, min(args.steps, 30))
        return
    if args.graph:
        graph_bench(dev, max(args.steps, 100))
        return
    if args.configs:
        configs_bench(dev, min(args.steps, 10))
        return
    if args.bf16_state:
        probe_copies(dev, args.copy_probe_mib)
        state_storage_bench(dev, args.copies, min(args.steps, 30))
        return
    if args.norm:
        probe_copies(dev, args.copy_probe_mib)
        output_norm_bench(dev, args.copies, min(args.steps, 30))
        return
    print("[bench] generating inputs", file=sys.stderr, flush=True)

    pre = gs.workload("prefill")
    dec = gs.workload("decode", batch=B_DECODE)
    s_dec = gs.decode_state(B_DECODE, HV, D, D, seed=gs.SEED_BASE + 101)

    P = device_inputs(pre, dev)
    Dd = device_inputs(dec, dev)
    ws_bytes = gdn.prefill_workspace_size(1, T_PREFILL, HK, HV, D, D, CHUNK, torch.bfloat16)
    sets = []
    for i in range(args.copies):
        sets.append(dict(
            q=P["q"].clone(), k=P["k"].clone(), v=P["v"].clone(), g=P["g"].clone(),
            beta=P["beta"].clone(), cu=P["cu_seqlens"].clone(),
            out=torch.empty((T_PREFILL, HV, D), dtype=torch.bfloat16, device=dev),
            fin=torch.empty((1, HV, D, D), dtype=torch.float32, device=dev),
            ws=torch.empty(ws_bytes, dtype=torch.uint8, device=dev),
            dq=Dd["q"].clone(), dk=Dd["k"].clone(), dv=Dd["v"].clone(), dg=Dd["g"].clone(),
            db=Dd["beta"].clone(), state=torch.from_numpy(s_dec).to(dev),
            dout=torch.empty((B_DECODE, HV, D), dtype=torch.bfloat16, device=dev),
        ))

    def step(s):
        gdn.prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu"], chunk=CHUNK,
                    final_state=s["fin"], out=s["out"], workspace=s["ws"])
        gdn.decode_step(s["dq"], s["dk"], s["dv"], s["dg"], s["db"], s["state"], out=s["dout"])

    # ---- the GPU side of the parity check: one untimed step from fresh
    # decode states, its results copied to the host. The oracle runs on the
    # same inputs after the timed region; its comparison gates the output.
    s0 = sets[0]
    chk_state = torch.from_numpy(s_dec).to(dev)
    gdn.prefill(s0["q"], s0["k"], s0["v"], s0["g"], s0["beta"], s0["cu"], chunk=CHUNK,
                final_state=s0["fin"], out=s0["out"], workspace=s0["ws"])
    gdn.decode_step(s0["dq"], s0["dk"], s0["dv"], s0["dg"], s0["db"], chk_state, out=s0["dout"])
    torch.cuda.synchronize()

    def f64(t):
        return t.detach().to("cpu", torch.float64).numpy()

    gpu_check = {"prefill_out": f64(s0["out"]), "prefill_state": f64(s0["fin"]),
                 "decode_out": f64(s0["dout"]), "decode_state": f64(chk_state)}
    del chk_state

    stream = torch.cuda.current_stream(dev)
    probe_copies(dev, args.copy_probe_mib)

    # ---- measurement passes, each over --steps steps, before the timed
    # region: they run right before it, so that the timed steps do not start
    # on a GPU whose clocks dropped while it idled (measured after an 8 s
    # pause: 157 us per step after 10 warm-up steps, 149 us after 100).
    # spread of the step time (an event pair per step)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(sets[i % args.copies])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) for a, b in evs)

    def pct(p):
        return per_step[min(len(per_step) - 1, int(round(p / 100 * (len(per_step) - 1))))]

    # prefill-only and decode-only rates
    def timed(fn, n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            fn(sets[i % args.copies])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    ms_pre = timed(lambda s: gdn.prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu"], chunk=CHUNK,
                                         final_state=s["fin"], out=s["out"], workspace=s["ws"]), args.steps)
    ms_dec = timed(lambda s: gdn.decode_step(s["dq"], s["dk"], s["dv"], s["dg"], s["db"], s["state"],
                                             out=s["dout"]), args.steps)

    # each kernel's duration (every launch stamped by its own dispatch), last,
    # on clocks the passes above have brought up
    gdn.timing_start(8 * args.steps)
    for i in range(args.steps):
        step(sets[i % args.copies])
    kt = gdn.timing_stop()
    torch.cuda.synchronize()


    # ---- warm-up, then the timed region: exactly --steps steps
    for i in range(args.warmup):
        step(sets[i % args.copies])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(sets[i % args.copies])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / args.steps

    # ---- the oracle on the same inputs (this is also the CPU baseline) and
    # the parity gate: no throughput is reported unless the checked step
    # matches it.
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    threads = max(1, min(16, ncpu))
    print("[bench] oracle reference (and CPU baseline)", file=sys.stderr, flush=True)
    cpu_rec, ref = cpu_baseline(pre, dec, s_dec, threads, one_thread=not args.no_cpu_baseline)
    errs = parity_errors(gpu_check, ref)
    parity = {"max_rel_err": errs, "bars": PARITY_BARS,
              "pass": all(errs[k] <= PARITY_BARS[k] for k in PARITY_BARS),
              "reference": "fp64 oracle, every token and value head of the timed step's inputs"}
    if not parity["pass"]:
        print(json.dumps({"metric": METRIC, "error": "parity gate failed: the GPU step does not match "
                          "the oracle; no throughput is reported", "parity": parity}), flush=True)
        sys.exit(1)

    scan_ms = kt["scan"]["mean_ms"]
    prep_ms = kt["prep"]["mean_ms"]
    dec_ms = kt["decode"]["mean_ms"]
    scan_flops = scan_flops_per_token() * T_PREFILL
    prep_flops = prep_flops_per_token() * T_PREFILL
    scan_tflops = scan_flops / (scan_ms * 1e-3) / 1e12
    dec_bytes = decode_bytes_per_step()
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9

    sched_ms = kt["schedule"]["mean_ms"] if kt["schedule"]["count"] else 0.0
    prefill_kernel_ms = sched_ms + prep_ms + scan_ms
    prefill_all_flops = scan_flops + prep_flops
    pre_tflops = prefill_all_flops / (prefill_kernel_ms * 1e-3) / 1e12
    t_prep, t_scan = measured_traffic("gdn_prep_kernel"), measured_traffic("gdn_scan_kernel")
    # The headline is the whole prefill (its kernels, launched back to back on
    # one stream, as one launch of the layer): the chunked form's algorithmic
    # MFMA flops per prefill over the summed mean durations of its kernels.
    roof = {"bound": "mfma", "kernel": "prefill (gdn_prep_kernel + gdn_scan_kernel)", "achieved": pre_tflops,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": pre_tflops / PEAK_BF16_TFLOPS,
            "traffic": None if t_prep is None or t_scan is None else t_prep + t_scan,
            "algorithmic_per_launch": prefill_all_flops, "mean_launch_ms": prefill_kernel_ms,
            "kernel_mean_ms": {"schedule": sched_ms, "prep": prep_ms, "scan": scan_ms},
            "target_frac": 0.40}
    roof_scan = {"bound": "mfma", "kernel": "gdn_scan_kernel", "achieved": scan_tflops,
                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": scan_tflops / PEAK_BF16_TFLOPS,
                 "traffic": t_scan, "algorithmic_per_launch": scan_flops, "mean_launch_ms": scan_ms}
    roof_dec = {"bound": "hbm", "kernel": "gdn_decode_kernel", "achieved": dec_gbs, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": dec_gbs / PEAK_HBM_GBS,
                "traffic": measured_traffic("gdn_decode_kernel"),
                "algorithmic_per_launch": dec_bytes, "mean_launch_ms": dec_ms}
    res = {
        "metric": METRIC,
        "value": (T_PREFILL + B_DECODE) / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"GDN layer step: prefill 1x{T_PREFILL} tokens + decode batch {B_DECODE}; "
                               f"HK={HK}, HV={HV}, d={D}, chunk {CHUNK}; bf16 q/k/v/out, fp32 gates/state",
                   "prefill_tokens": T_PREFILL, "decode_batch": B_DECODE, "parallelism": "single GPU",
                   "buffer_copies": args.copies},
        "roofline": roof,
        "roofline_scan": roof_scan,
        "roofline_decode": roof_dec,
        "prefill": {"tokens_per_s": T_PREFILL / (ms_pre * 1e-3), "ms": ms_pre,
                    "mfma_frac_all_kernels": prefill_all_flops / (ms_pre * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                    "kernel_ms": {"schedule": kt["schedule"]["mean_ms"], "prep": prep_ms, "scan": scan_ms}},
        "decode": {"tokens_per_s": B_DECODE / (ms_dec * 1e-3), "ms": ms_dec, "kernel_ms": dec_ms,
                   "hbm_frac": dec_gbs / PEAK_HBM_GBS},
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "step_ms_percentiles": {"p10": pct(10), "p50": pct(50), "p90": pct(90)},
        "kernel_source_hash": kernel_source_hash(),
    }
    res["parity"] = parity
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_rec
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
