#!/usr/bin/env python3
"""Benchmark of the SQuad-Attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps 150] [--warmup 5]

One step is one squad_attn_fwd call (local pass, then global pass) over the
Wan 2.2 5B-shaped block at 704x1280x81: n = 18,480 tokens (grid 21x22x40),
24 heads of dim 128, window 21x2x4 (168 tokens, 110 windows), bf16.  Inputs are
seeded synthetic tensors of that shape already resident in HBM; two complete
input/output sets are used alternately so that the 256 MB last-level cache
cannot hold a whole set between steps.

Prints one JSON line: effective TFLOP/s (algorithmic FLOPs 4*B*h*d*n*(m+N_w)
per step over the measured time) plus ms per block, a roofline object for the
dominant kernel (its own launches timed with HIP events on the launch stream)
and the oracle's throughput on the host cores (a bounded sample).
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PAGES_MS_PER_BLOCK = 4.27      # the pages' SQuad attention latency per block (H100, bf16, n = 18,480)
KERNEL_SOURCES = ["sub_quadratic_factorized_amd/csrc/squad_pass_bf16.hip",
                  "sub_quadratic_factorized_amd/csrc/squad_internal.h",
                  "sub_quadratic_factorized_amd/csrc/squad_layout.h"]
# rocprofv3 runs whose CSV output --summarize-profiles turns into the files under profiles/
PROFILE_ARGS = "--no-cpu-baseline --no-other-workloads --steps 20 --warmup 2 --kernel-iters 20 --copy-calibration-mib 512"
# counter passes (each within the per-block limits of one rocprofv3 run)
COUNTER_PASSES = {
    "mfma_lds": "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_LDS "
                "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INSTS_VALU SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "waits": "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_ANY "
             "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM GRBM_GUI_ACTIVE",
    "rdreq": "TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum",
    "wrreq": "TCC_BUBBLE_sum TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum",
}
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d <out>/trace -o run -- python3 bench.py " + PROFILE_ARGS,
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d <out>/fetch -o run -- python3 bench.py " + PROFILE_ARGS,
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d <out>/write -o run -- python3 bench.py " + PROFILE_ARGS,
}
for _name, _ctrs in COUNTER_PASSES.items():
    PROFILE_COMMANDS[_name] = (f"rocprofv3 --pmc {_ctrs} -f csv -d <out>/{_name} -o run -- python3 bench.py "
                               + PROFILE_ARGS)
PASS_KERNELS = {"squad_local_pass": "squad_local_pass_bf16", "squad_global_pass": "squad_global_pass_bf16"}


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and whitespace removed, so that
    only a change of the code itself invalidates the stored counters."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def time_loop(fn, iters, sets, warmup=2):
    """Average ms per call of fn(set) over `iters` calls, HIP events on the current stream."""
    import torch
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(iters):
        fn(sets[i % len(sets)])
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def short_kernel_name(name: str) -> str:
    """Kernel name without return type, namespaces and parameter list (template arguments kept)."""
    name = name.strip('"')
    if name.startswith("void "):
        name = name[5:]
    depth, cut = 0, len(name)
    for i, ch in enumerate(name):  # the parameter list is the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not name.startswith("(anonymous", i):
            cut = i
            break
    name = name[:cut]
    base, _, targs = name.partition("<")
    base = base.split("::")[-1]
    return base + ("<" + targs if targs else "")


MI355X_XCDS = 8          # GRBM_GUI_ACTIVE in the counter CSV is summed over the XCDs
MI355X_SIMDS = 256 * 4   # 256 CUs of 4 SIMDs


def _counter_means(d: str):
    """{(kernel, counter): (mean value per dispatch, dispatches)} of one rocprofv3 --pmc run's CSV."""
    import csv
    vals = {}
    for row in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        key = (short_kernel_name(row["Kernel_Name"]), row["Counter_Name"])
        vals.setdefault(key, []).append(float(row["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def _kernels_with(means, counter):
    return sorted({k for k, c in means if c == counter})


def summarize_profiles(prof_dir: str, workload: str, trace_log: str | None = None) -> None:
    """Write the profiles/ summaries from one folder holding the CSV output of
    every PROFILE_COMMANDS run (one subfolder per run, named as its key).

    HBM bytes come from the read and write request counts by size
    (TCC_EA0_RDREQ_32B/64B/128B, TCC_EA0_WRREQ and _64B) times their sizes, with
    no fitted factor; FETCH_SIZE and WRITE_SIZE are listed beside them for the
    plain device copy the same runs make (its bytes are known)."""
    import csv
    from sub_quadratic_factorized_amd import workloads as wl
    w = wl.WORKLOADS[workload]
    esize = 2 if w.dtype == "bf16" else 4
    tensor = w.B * w.n * w.heads * w.d * esize
    pass_bytes = 4 * tensor
    copy_bytes = 512 << 20
    sub = {k: os.path.join(prof_dir, k) for k in PROFILE_COMMANDS}
    rd, wr = _counter_means(sub["rdreq"]), _counter_means(sub["wrreq"])
    fetch, write = _counter_means(sub["fetch"]), _counter_means(sub["write"])
    ml, wt = _counter_means(sub["mfma_lds"]), _counter_means(sub["waits"])

    def hbm(kernel):
        g = lambda m, c: m.get((kernel, c), (0.0, 0))[0]
        n128, n64, n32 = g(rd, "TCC_EA0_RDREQ_128B_sum"), g(rd, "TCC_EA0_RDREQ_64B_sum"), g(rd, "TCC_EA0_RDREQ_32B_sum")
        nall = g(rd, "TCC_EA0_RDREQ_sum")
        w64, wall = g(wr, "TCC_EA0_WRREQ_64B_sum"), g(wr, "TCC_EA0_WRREQ_sum")
        return (128 * n128 + 64 * n64 + 32 * n32, 64 * w64 + 32 * (wall - w64),
                nall - n128 - n64 - n32, g(wr, "TCC_BUBBLE_sum"))

    stats = []
    for row in csv.DictReader(open(os.path.join(sub["trace"], "run_kernel_stats.csv"))):
        stats.append((short_kernel_name(row["Name"]), int(row["Calls"]), float(row["AverageNs"]) / 1e3,
                      float(row["MinNs"]) / 1e3, float(row["MaxNs"]) / 1e3))
    avg_us = lambda k: next((s[2] for s in stats if s[0] == k), float("nan"))
    title = (f"{w.name}: B={w.B}, grid {w.T}x{w.Hs}x{w.Ws} (n={w.n}), {w.heads} heads, d={w.d}, "
             f"window {w.wt}x{w.wh}x{w.ww} (m={w.m}, N_w={w.n_windows}), {w.dtype}")
    src_hash = kernel_source_hash()
    wl_arg = "" if w.name == wl.HEADLINE else f" --workload {w.name}"
    cmd = lambda k: PROFILE_COMMANDS[k] + wl_arg
    intro = ("Commands (repository root on one MI355X, `export TMPDIR=/tmp` first; <out> any scratch folder; "
             "each counter pass is a run of its own):\n\n```\n")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    out = lambda name: open(os.path.join(ROOT, "profiles", f"{name}_{w.name}.md"), "w")

    with out("kernel_trace_squad_passes") as f:
        f.write(f"# Kernel trace: SQuad-Attention passes, {title}\n\n" + intro + cmd("trace") + "\n```\n\n")
        f.write(f"Kernel source hash (bench.py kernel_source_hash): {src_hash}\n\n")
        f.write("| kernel | calls | average (us) | min (us) | max (us) |\n|---|---|---|---|---|\n")
        for name, calls, avg, lo, hi in stats:
            shown = name if len(name) <= 72 else name[:69] + "..."
            f.write(f"| {shown} | {calls} | {avg:.1f} | {lo:.1f} | {hi:.1f} |\n")
        if trace_log:
            own = [ln.strip() for ln in open(trace_log) if ln.startswith("[bench] ") and " ms" in ln]
            f.write("\nbench.py's own HIP-event timings in the same profiled process (stderr):\n\n```\n"
                    + "\n".join(own) + "\n```\n")

    copy = next(k for k, c in rd if c == "TCC_EA0_RDREQ_sum" and "copyBuffer" in k)
    c_rd, c_wr, c_other, c_bubble = hbm(copy)
    c_fetch = fetch.get((copy, "FETCH_SIZE"), (0.0, 0))[0] * 1024
    c_write = write.get((copy, "WRITE_SIZE"), (0.0, 0))[0] * 1024
    rows, brows = [], []
    for kname, prefix in PASS_KERNELS.items():
        kern = next(k for k in _kernels_with(rd, "TCC_EA0_RDREQ_sum") if k.startswith(prefix))
        r, wbytes, _, _ = hbm(kern)
        rec = {"kernel": kname, "instance": kern, "workload": w.name,
               "hbm_read_bytes_per_launch": r, "hbm_write_bytes_per_launch": wbytes,
               "hbm_bytes_per_launch": r + wbytes, "algorithmic_bytes_per_launch": pass_bytes,
               "method": "read requests x their sizes (TCC_EA0_RDREQ_128B/64B/32B) + write requests x "
                         "their sizes (TCC_EA0_WRREQ, _64B), mean per dispatch",
               "kernel_source_hash": src_hash, "commands": [cmd("rdreq"), cmd("wrreq")]}
        with open(os.path.join(ROOT, "profiles", f"traffic_{kname}_{w.name}.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        t = avg_us(kern)
        rows.append(f"| {kern} | {r / 1e6:.1f} | {wbytes / 1e6:.1f} | {(r + wbytes) / 1e6:.1f} | "
                    f"{pass_bytes / 1e6:.1f} | {(r + wbytes) / pass_bytes:.3f} | {t:.1f} | "
                    f"{(r + wbytes) / t / 1e3:.0f} |")
    # the backward's kernels: the global pass's backward reads q, k, Y, O, dO and writes dY and its dq,
    # dk contributions (8 tensor-sizes); the local pass's reads q, k, v, dY and those contributions
    # and writes dq, dk, dv (9); per-row float32 arrays not counted
    for prefix, alg, what in (("squad_bwd_pass_bf16<128, false", 8 * tensor, "global pass"),
                              ("squad_bwd_onesweep_bf16<128", 9 * tensor, "local pass, one sweep"),
                              ("squad_bwd_pass_bf16<128, true", 9 * tensor, "local pass")):
        kern = next((k for k in _kernels_with(rd, "TCC_EA0_RDREQ_sum") if k.startswith(prefix)), None)
        if kern is None:
            continue
        r, wbytes, _, _ = hbm(kern)
        t = avg_us(kern)
        brows.append(f"| {kern} ({what}) | {r / 1e6:.1f} | {wbytes / 1e6:.1f} | {(r + wbytes) / 1e6:.1f} | "
                     f"{alg / 1e6:.1f} | {(r + wbytes) / alg:.3f} | {t:.1f} | {(r + wbytes) / t / 1e3:.0f} |")
    head = ("| kernel | HBM read (MB) | HBM write (MB) | total (MB) | algorithmic (MB) | ratio | "
            "trace avg (us) | GB/s |\n|---|---|---|---|---|---|---|---|\n")
    with out("hbm_traffic_squad_passes") as f:
        f.write(f"# HBM traffic per launch: SQuad-Attention passes, {title}\n\n" + intro + cmd("rdreq") + "\n"
                + cmd("wrreq") + "\n" + cmd("fetch") + "\n" + cmd("write") + "\n" + cmd("trace") + "\n```\n\n")
        f.write(f"Kernel source hash: {src_hash}\n\n")
        f.write("Bytes = read requests times their sizes (TCC_EA0_RDREQ_128B, _64B, _32B) plus write requests "
                "times theirs (TCC_EA0_WRREQ, of which _64B), mean per dispatch; no scale factor.\n\n")
        f.write(f"Cross-check on the plain {copy_bytes >> 20} MiB device copy of the same runs ({copy}): "
                f"requests read {c_rd / 2**20:.1f} MiB and write {c_wr / 2**20:.1f} MiB "
                f"({int(round(c_other))} read requests of other sizes). FETCH_SIZE reads {c_fetch / 2**20:.1f} MiB and "
                f"WRITE_SIZE {c_write / 2**20:.1f} MiB for it: FETCH_SIZE's expression counts 128-byte reads "
                f"through TCC_BUBBLE (here {c_bubble:.0f}) and every other non-32-byte read as 64 bytes, so on "
                f"this part, where reads go out as 128-byte requests and TCC_BUBBLE stays 0, it reports half "
                f"the bytes read.\n\n")
        f.write(head + "\n".join(rows) + "\n")
    if brows:
        with out("hbm_traffic_squad_backward") as f:
            f.write(f"# HBM traffic per launch: SQuad-Attention backward kernels, {title}\n\n"
                    "From the same counter runs as the passes' summary (the runs time squad_attn_bwd and "
                    "squad_attn_bwd_saved after the forward), bytes from request counts by size:\n\n```\n"
                    + cmd("rdreq") + "\n" + cmd("wrreq") + "\n```\n\n")
            f.write("Algorithmic bytes: the global pass's backward reads q, k, Y, O and dO and writes dY and "
                    "its dq, dk contributions (8 tensor-sizes); the local pass's reads q, k, v, dY and those "
                    "contributions and writes dq, dk, dv (9); per-row float32 arrays not counted.\n\n")
            f.write(head + "\n".join(brows) + "\n")

    # MFMA, LDS and wave states per kernel
    mrows = []
    flops_alg = {"squad_local_pass": 4 * w.B * w.heads * w.d * w.n * w.m,
                 "squad_global_pass": 4 * w.B * w.heads * w.d * w.n * w.n_windows}
    kernels = [k for k in _kernels_with(ml, "SQ_INSTS_VALU_MFMA_MOPS_BF16") if "squad" in k]
    for kern in kernels:
        g = lambda m, c: m.get((kern, c), (0.0, 0))[0]
        cyc = g(ml, "GRBM_GUI_ACTIVE") / MI355X_XCDS
        busy = g(ml, "SQ_VALU_MFMA_BUSY_CYCLES") / max(cyc * MI355X_SIMDS, 1.0)
        flops = g(ml, "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
        t = avg_us(kern)
        lds_active = g(ml, "SQ_LDS_IDX_ACTIVE")
        conflict = g(ml, "SQ_LDS_BANK_CONFLICT") / lds_active if lds_active else 0.0
        wave = g(wt, "SQ_WAVE_CYCLES")
        frac = lambda c: g(wt, c) / wave if wave else 0.0
        alg = next((v for k2, v in flops_alg.items() if kern.startswith(PASS_KERNELS[k2])), None)
        mrows.append(
            f"| {kern} | {t:.1f} | {flops / 1e9:.2f} | {'' if alg is None else f'{alg / 1e9:.2f}'} | "
            f"{flops / t / 1e6:.0f} | {100 * busy:.1f} | {g(ml, 'SQ_INSTS_MFMA') / 1e6:.2f} | "
            f"{g(ml, 'SQ_INSTS_VALU') / 1e6:.2f} | {g(ml, 'SQ_INSTS_LDS') / 1e6:.2f} | {100 * conflict:.1f} | "
            f"{100 * frac('SQ_ACTIVE_INST_ANY'):.0f} | {100 * frac('SQ_WAIT_INST_ANY'):.0f} | "
            f"{100 * frac('SQ_WAIT_ANY'):.0f} | {100 * frac('SQ_WAIT_INST_LDS'):.0f} |")
    with out("mfma_lds_squad_passes") as f:
        f.write(f"# MFMA, LDS and wave states per launch: SQuad-Attention kernels, {title}\n\n" + intro
                + cmd("mfma_lds") + "\n" + cmd("waits") + "\n" + cmd("trace") + "\n```\n\n")
        f.write(f"Kernel source hash: {src_hash}\n\n")
        f.write("Per dispatch, mean over the runs' dispatches. MFMA FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 "
                "(the work the MFMAs did, padded tiles and the row-sum MFMA included); algorithmic = "
                "4 B h d n L of the pass. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x "
                f"{MI355X_SIMDS} SIMDs). Instruction counts are wave instructions (millions). LDS conflict = "
                "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE. Wave states are shares of SQ_WAVE_CYCLES: "
                "issuing (SQ_ACTIVE_INST_ANY), waiting to issue (SQ_WAIT_INST_ANY), waiting on a counter "
                "(SQ_WAIT_ANY, s_waitcnt and barriers), of which for LDS (SQ_WAIT_INST_LDS). MFMA peak: "
                f"{BF16_MFMA_PEAK_TFLOPS:.0f} TFLOP/s dense bf16.\n\n")
        f.write("| kernel | trace avg (us) | MFMA GFLOP | algorithmic GFLOP | MFMA TFLOP/s | MFMA busy % | "
                "MFMA instr (M) | VALU instr (M) | LDS instr (M) | LDS conflict % | active % | wait-issue % | "
                "wait-counter % | wait LDS % |\n|---|---|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        f.write("\n".join(mrows) + "\n")


# Backbones of the FLOP-conformance sweep: native latent grid (81 frames, T = 21)
# and attention heads x head dim (Wan 2.2 5B at 704x1280; Wan 2.1 1.3B and 14B at
# 480x832).
SWEEP_BACKBONES = {"5B": ((22, 40), 24), "1.3B": ((30, 52), 12), "14B": ((30, 52), 40)}


def sweep_grids(native, count=10, span=30.0):
    """`count` grids at the native aspect ratio with T = 21 whose token counts
    grow geometrically over `span` (from 1/6 to 5 times the native n)."""
    Hs0, Ws0 = native
    out = []
    for i in range(count):
        s = ((1.0 / 6.0) * span ** (i / (count - 1))) ** 0.5
        out.append((21, max(2, round(Hs0 * s)), max(2, round(Ws0 * s))))
    return out


def run_sweep(iters: int) -> None:
    """One JSON line per (backbone, grid): the window rule's window, the
    closed-form FLOPs on the padded grid against the 8hd n^1.5 optimum, and the
    measured time of squad_attn_fwd_padded (bf16, d = 128, synthetic inputs)."""
    import torch
    from sub_quadratic_factorized_amd import binding as bd
    d = 128
    for name, (native, heads) in SWEEP_BACKBONES.items():
        for grid in sweep_grids(native):
            T, Hs, Ws = grid
            win = bd.squad_window_solve(grid)
            n = T * Hs * Ws
            flops = bd.squad_attn_flops_padded(1, heads, *grid, *win, d)
            optimum = 8.0 * heads * d * n ** 1.5
            gen = torch.Generator(device="cuda")
            gen.manual_seed(n)  # seeded N(0, 1) drawn on the device: timing only, no parity here
            q, k, v = (torch.randn((1, n, heads, d), generator=gen, device="cuda").to(torch.bfloat16)
                       for _ in range(3))
            need = bd.squad_attn_padded_workspace_bytes(1, heads, *grid, *win, d, bd.SQUAD_BF16)
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            out = torch.empty_like(q)
            ms = time_loop(lambda s: bd.squad_attn_fwd_padded(q, k, v, grid, win, out=out, workspace=ws),
                           iters, [None])
            _, Hp, Wp = (T, -(-Hs // win[1]) * win[1], -(-Ws // win[2]) * win[2])
            rec = {"backbone": name, "heads": heads, "grid": list(grid), "n": n, "window": list(win),
                   "padded_grid": [T, Hp, Wp], "closed_form_tflops": flops / 1e12,
                   "over_optimum": flops / optimum - 1.0, "ms": ms, "tflops_per_s": flops / (ms * 1e-3) / 1e12,
                   "algorithmic_gbs": bd.squad_attn_bytes_padded(1, heads, *grid, *win, d, bd.SQUAD_BF16)
                   / (ms * 1e-3) / 1e9}
            print(json.dumps(rec), flush=True)
            del q, k, v, ws, out
        torch.cuda.empty_cache()


def blas_description():
    """(name, threads) of the BLAS library numpy's products run on, as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover - threadpoolctl is optional
        libs = []
    if not libs:
        return "unknown", None
    i = libs[0]
    name = f"{i.get('internal_api', '?')} {i.get('version', '?')} ({os.path.basename(i.get('filepath', '?'))})"
    return name, i.get("num_threads")


def cpu_baseline(w, runs=3):
    """The fp64 oracle on the host cores: the whole block (every head of batch
    element 0) timed as 1 untimed warm-up run plus the minimum of `runs` timed
    runs, BLAS threads set to the cores this process may run on."""
    from oracle import squad_oracle as so
    from sub_quadratic_factorized_amd import workloads as wl
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl is optional
        limiter = None
    blas, blas_threads = blas_description()
    table = so.window_slot_table(w.T, w.Hs, w.Ws, w.wt, w.wh, w.ww)
    per_head_flops = so.squad_flops(1, 1, w.T, w.Hs, w.Ws, w.wt, w.wh, w.ww, w.d)
    heads = [wl.head_slices_f64(w, 0, h) for h in range(w.heads)]  # generated untimed
    times = []
    for r in range(runs + 1):
        t0 = time.perf_counter()
        for q, k, v in heads:
            so.squad_head(q, k, v, table)
        if r > 0:  # run 0 is the warm-up
            times.append(time.perf_counter() - t0)
    if limiter is not None:
        limiter.unregister()
    best = min(times)
    return {
        "value": len(heads) * per_head_flops / best / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"the {w.heads} heads of batch element 0 of {w.name} (the whole block at B = 1), numpy float64; "
                  f"1 warm-up run, then the minimum of {runs} runs",
        "blas": blas,
        "blas_threads": blas_threads,
        "runs_s": times,
        "ms_per_block_equiv": best / len(heads) * w.B * w.heads * 1e3,
    }


def time_other_workload(name, steps=20, warmup=5, kernel_iters=10, spin_up_s=0.3):
    """One of the other configurations, timed like the headline (a single
    input set: each of these sets exceeds the last-level cache on its own;
    the tiny fp32 case is launch-bound and reported in ms only)."""
    import torch
    from sub_quadratic_factorized_amd import binding as bd
    from sub_quadratic_factorized_amd import workloads as wl
    w = wl.WORKLOADS[name]
    grid, window = (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww)
    dt = bd.SQUAD_BF16 if w.dtype == "bf16" else bd.SQUAD_F32
    flops = bd.squad_attn_flops(*w.geometry())
    nbytes = bd.squad_attn_bytes(*w.geometry(), dt)
    t0 = time.perf_counter()
    q, k, v = wl.device_inputs(w, seed=0)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    gen_s = time.perf_counter() - t0
    sets = [(q, k, v, out)]

    def step(s):
        bd.squad_attn_fwd(s[0], s[1], s[2], grid, window, out=s[3])

    # the GPU idled while the inputs were generated: untimed steps for
    # spin_up_s bring its clocks back up, then the warm-up
    t_spin = time.perf_counter()
    while time.perf_counter() - t_spin < spin_up_s:
        for _ in range(5):
            step(sets[0])
        torch.cuda.synchronize()
    for _ in range(warmup):
        step(sets[0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(sets[0])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    local_ms = time_loop(lambda s: bd.squad_attn_local(s[0], s[1], s[2], grid, window, out=s[3]), kernel_iters, sets)
    global_ms = time_loop(lambda s: bd.squad_attn_global(s[0], s[1], s[3], grid, window, out=s[3]),
                          kernel_iters, sets)
    rec = {"config": {"B": w.B, "heads": w.heads, "d": w.d, "grid": list(grid), "window": list(window), "n": w.n,
                      "m": w.m, "n_windows": w.n_windows}, "dtype": w.dtype, "steps": steps, "warmup": warmup,
           "ms_per_block": ms, "local_pass_ms": local_ms, "global_pass_ms": global_ms}
    if w.dtype == "bf16":
        gbs = nbytes / (ms * 1e-3) / 1e9
        rec.update({"effective_tflops": flops / (ms * 1e-3) / 1e12, "algorithmic_gbs": gbs,
                    "fraction_of_roofline": gbs / HBM_PEAK_GBS,
                    "local_pass_frac": nbytes / 2 / (local_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "global_pass_frac": nbytes / 2 / (global_ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
    eprint(f"[bench] {name}: {ms:.4f} ms/block (local {local_ms:.4f}, global {global_ms:.4f}; "
           f"inputs generated in {gen_s:.1f} s)")
    del q, k, v, out, sets
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=150)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: the 5B 704p block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the other configurations' figures (other_workloads in the JSON line)")
    ap.add_argument("--kernel-iters", type=int, default=100)
    ap.add_argument("--spin-up-s", type=float, default=0.3,
                    help="untimed steps for this many seconds before the warm-up (GPU clocks to steady state)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this size (for scaling hardware byte counters)")
    ap.add_argument("--summarize-profiles", metavar="PROF_DIR",
                    help="write the profiles/ summaries from rocprofv3 CSV output, then exit (no GPU needed)")
    ap.add_argument("--trace-log", default=None, help="stderr of the profiled trace run (with --summarize-profiles)")
    ap.add_argument("--sweep", action="store_true",
                    help="the window-rule sweep (10 grids x 3 backbones, padded entry point): one JSON line per grid")
    args = ap.parse_args()

    if args.summarize_profiles:
        from sub_quadratic_factorized_amd import workloads as wl
        summarize_profiles(args.summarize_profiles, args.workload or wl.HEADLINE, args.trace_log)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sub_quadratic_factorized_amd import binding as bd
    from sub_quadratic_factorized_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    bd.lib()  # fail loudly if the HIP library is missing

    if args.sweep:
        run_sweep(max(args.kernel_iters // 5, 5))
        return

    w = wl.WORKLOADS[args.workload or wl.HEADLINE]
    grid, window = (w.T, w.Hs, w.Ws), (w.wt, w.wh, w.ww)
    flops = bd.squad_attn_flops(*w.geometry())
    dt = bd.SQUAD_BF16 if w.dtype == "bf16" else bd.SQUAD_F32
    bytes_fwd = bd.squad_attn_bytes(*w.geometry(), dt)
    pass_bytes = bytes_fwd / 2  # each pass reads three tensors and writes one

    eprint(f"[bench] workload {w.name}: generating inputs")
    q, k, v = wl.device_inputs(w, seed=0)
    sets = [(q, k, v, torch.empty_like(q))]
    # a second, different set (rotated inputs keep the last-level cache honest)
    sets.append((q.roll(1, dims=2).contiguous(), k.roll(1, dims=2).contiguous(), v.roll(1, dims=2).contiguous(),
                 torch.empty_like(q)))
    torch.cuda.synchronize()

    def step(s):
        bd.squad_attn_fwd(s[0], s[1], s[2], grid, window, out=s[3])

    # ---- untimed spin-up, then W warm-up steps --------------------------------
    # The GPU sat idle while inputs were generated; a few hundred milliseconds
    # of steps bring it to its steady clocks (measured: the first timed loop
    # otherwise runs up to 15 % slow).  Like the warm-up, none of it is timed.
    t_spin = time.perf_counter()
    while time.perf_counter() - t_spin < args.spin_up_s:
        for i in range(20):
            step(sets[i % 2])
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(sets[i % 2])
    torch.cuda.synchronize()

    # ---- the timed region: exactly `steps` forward passes, back to back -------
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    region[0].record()
    for i in range(args.steps):
        step(sets[i % 2])
    region[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    region_ms = region[0].elapsed_time(region[1]) / args.steps

    # per-step spread (not the timed region: an event pair around every step
    # adds work to the stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        step(sets[i % 2])
        ev[i][1].record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    mean_ms = sum(per) / len(per)
    eprint(f"[bench] fwd: wall {ms_per_step:.4f} ms/step (stream events {region_ms:.4f}); per-step events mean "
           f"{mean_ms:.4f} median {per[len(per)//2]:.4f} min {per[0]:.4f} ms")

    # warm (single set) figure for reference
    warm_ms = time_loop(step, args.kernel_iters, sets[:1])

    # ---- per-kernel timing for the roofline ---------------------------------
    def local(s):
        bd.squad_attn_local(s[0], s[1], s[2], grid, window, out=s[3])

    def glob(s):
        bd.squad_attn_global(s[0], s[1], s[3], grid, window, out=s[3])

    def reversed_order(s):
        bd.squad_attn_fwd_reversed(s[0], s[1], s[2], grid, window, out=s[3])

    local_ms = time_loop(local, args.kernel_iters, sets)
    global_ms = time_loop(glob, args.kernel_iters, sets)
    reversed_ms = time_loop(reversed_order, max(args.kernel_iters // 5, 5), sets)
    eprint(f"[bench] local pass {local_ms:.4f} ms/launch, global pass {global_ms:.4f} ms/launch, warm fwd {warm_ms:.4f}")
    dom, dom_ms = ("local", local_ms) if local_ms >= global_ms else ("global", global_ms)
    kname = "squad_local_pass" if dom == "local" else "squad_global_pass"
    achieved = pass_bytes / (dom_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(kname, w.name)

    value = flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": "SQuad attn ms/block + effective TFLOP/s & % roofline, n=18480 h=24 d=128 bf16",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": PAGES_MS_PER_BLOCK / ms_per_step if w.name == wl.HEADLINE else None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "heads": w.heads, "d": w.d, "grid": list(grid), "window": list(window),
            "n": w.n, "m": w.m, "n_windows": w.n_windows, "input_sets_rotated": 2,
        },
        "ms_per_block": {"wall_mean": ms_per_step, "region_events_mean": region_ms,
                         "event_mean": mean_ms, "event_median": per[len(per) // 2],
                         "event_min": per[0], "warm_single_set": warm_ms},
        "effective_tflops": value,
        "algorithmic_gbs": bytes_fwd / (ms_per_step * 1e-3) / 1e9,
        "fraction_of_roofline": (bytes_fwd / (ms_per_step * 1e-3) / 1e9) / HBM_PEAK_GBS,
        "kernels_ms": {"squad_local_pass": local_ms, "squad_global_pass": global_ms},
        "reversed_order_ms": reversed_ms,
        "roofline": {
            "kernel": kname,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": pass_bytes,
            "mfma_tflops": (flops * (w.m if dom == "local" else w.n_windows) / (w.m + w.n_windows))
                           / (dom_ms * 1e-3) / 1e12,
            "mfma_peak_tflops": BF16_MFMA_PEAK_TFLOPS,
        },
        "baseline_context": {"pages_ms_per_block": PAGES_MS_PER_BLOCK, "hardware": "NVIDIA H100 80GB (pages)"},
        "kernel_source_hash": kernel_source_hash(),
    }
    # ---- the gradients of the same call (squad_attn_bwd), same inputs ---------
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    dout = wl.device_inputs(w, seed=1)[0]
    ws = torch.empty(bd.squad_attn_bwd_workspace_bytes(*w.geometry(), dt), dtype=torch.uint8, device="cuda")

    def bwd(s):
        bd.squad_attn_bwd(s[0], s[1], s[2], s[3], dout, grid, window, dq=dq, dk=dk, dv=dv, workspace=ws)

    bwd_ms = time_loop(bwd, max(args.kernel_iters // 5, 5), sets)
    bwd_flops = bd.squad_attn_bwd_flops(*w.geometry())
    bwd_bytes = bd.squad_attn_bwd_bytes(*w.geometry(), dt)
    eprint(f"[bench] backward {bwd_ms:.4f} ms ({bwd_flops / (bwd_ms * 1e-3) / 1e12:.1f} TFLOP/s)")
    out["backward"] = {"ms": bwd_ms, "tflops": bwd_flops / (bwd_ms * 1e-3) / 1e12, "flops": bwd_flops,
                       "kernel_bytes": bwd_bytes, "gbs": bwd_bytes / (bwd_ms * 1e-3) / 1e9,
                       "mfma_peak_frac": bwd_flops / (bwd_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                       "hbm_peak_frac": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    # ---- the same gradients from saved activations (squad_attn_fwd_save's Y
    # and log-sum-exp, made untimed per input set): no recomputation ---------
    del ws
    ws = torch.empty(bd.squad_attn_bwd_saved_workspace_bytes(*w.geometry(), dt), dtype=torch.uint8, device="cuda")
    saved = [bd.squad_attn_fwd_save(s[0], s[1], s[2], grid, window, out=s[3])[1:] for s in sets]
    which = {id(s): i for i, s in enumerate(sets)}

    def bwd_saved(s):
        y, lse = saved[which[id(s)]]
        bd.squad_attn_bwd_saved(s[0], s[1], s[2], s[3], dout, y, lse, grid, window, dq=dq, dk=dk, dv=dv,
                                workspace=ws)

    sv_ms = time_loop(bwd_saved, max(args.kernel_iters // 5, 5), sets)
    sv_bytes = bwd_bytes - 4.0 * w.B * w.n * w.heads * w.d * (2 if dt == bd.SQUAD_BF16 else 4)
    eprint(f"[bench] backward from saved activations {sv_ms:.4f} ms "
           f"({bwd_flops / (sv_ms * 1e-3) / 1e12:.1f} TFLOP/s)")
    out["backward_saved"] = {"ms": sv_ms, "tflops": bwd_flops / (sv_ms * 1e-3) / 1e12, "kernel_bytes": sv_bytes,
                             "gbs": sv_bytes / (sv_ms * 1e-3) / 1e9}
    del dq, dk, dv, dout, ws, saved

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = nbytes
        del src, dst
    if not args.no_other_workloads and w.name == wl.HEADLINE:
        del sets, q, k, v
        torch.cuda.empty_cache()
        out["other_workloads"] = {name: time_other_workload(name)
                                  for name in ("tiny_f32", "wan1p3b_480p", "wan5b_4x", "wan14b_4x_cfg")}
    if not args.no_cpu_baseline:
        eprint("[bench] timing the oracle on host cores (bounded sample)")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
