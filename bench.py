"""Benchmark of the sliding-window attention hot path on one MI355X.

One step = one pass of the whole path on Mistral-7B shapes:
  1. swa_prefill   causal, B=1, T=16384, W=4096, 32 query / 8 KV heads, d=128, bf16
  2. swa_cache_append  one new K/V row for each of 64 sequences (8 KV heads, d=128)
  3. swa_decode    64 sequences, 32/8 heads, d=128, full W=4096-slot rings,
                   positions uniform in [4096, 32768)
Inputs are seeded synthetic N(0,1) values rounded to bf16 (swa_inputs.py),
resident in HBM before timing starts.

Printed: one JSON line.  `value` is the in-window TFLOP/s of the whole step
(in-window FLOPs of prefill and decode, 4*d per (query, key) pair in a
window, over the step time); `parts` gives the prefill TFLOP/s against the
bf16 matrix peak and the decode KV-read GB/s against the HBM peak, each from
HIP events around its own launches; `roofline` describes the dominant kernel
(the prefill); `cpu_baseline` times the fp64 oracle on the host cores on a
bounded sample of the same work.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
       python bench.py --all-configs   (every configuration vs its roofline, warm and
                                        flushed; not the benchmark line)
       python bench.py --peaks         (the matrix-core and streaming-read rates this GPU
                                        sustains, from the library's calibration kernels)
       python bench.py --cpu-oracle    (the fp64 oracle's speed per configuration on the
                                        host cores, all threads and one)
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

import swa_inputs as si  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 matrix peak
METRIC = "SWA prefill in-window TFLOP/s + decode KV-read GB/s, % of MI355X peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_mistral7b_traffic.md")
COPY_BYTES = 256 << 20  # calibration copy: reads and writes this many bytes


def band_pairs_causal(T, W):
    """Number of (query, key) pairs inside causal windows of one head."""
    if T <= W:
        return T * (T + 1) // 2
    return W * (W + 1) // 2 + (T - W) * W


def prefill_work():
    c = si.WORKLOADS[3]
    pairs = band_pairs_causal(c["T"], c["W"]) * c["Hq"] * c["B"]
    flops = 4 * c["d"] * pairs
    elem = 2
    bytes_ = elem * c["T"] * c["d"] * c["B"] * (2 * c["Hq"] + 2 * c["Hkv"])  # Q, O, K, V
    return flops, bytes_


def decode_work(pos):
    c = si.WORKLOADS[4]
    rows = np.minimum(pos.astype(np.int64) + 1, c["W"]).sum()  # valid slots per sequence
    kv_bytes = int(rows) * c["Hkv"] * c["d"] * 2 * 2          # K and V, bf16
    qo_bytes = 2 * c["B"] * c["Hq"] * c["d"] * 2 + 4 * c["B"]
    flops = 4 * c["d"] * int(rows) * c["Hq"]
    return flops, kv_bytes, qo_bytes


def read_traffic(prefix, source):
    """HBM bytes per launch recorded in the committed counter summary under
    `<prefix>traffic_bytes_per_launch`, if it was taken on the current source
    of the kernel (`<prefix>traffic_kernel_sha256`)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    fields = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get(prefix + "traffic_kernel_sha256") != source_hash(source):
        return None
    try:
        return int(fields[prefix + "traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def source_hash(names):
    """SHA-256 of a kernel's source files' code: comments and whitespace
    removed, so that an edit of the comments alone keeps the measured figures
    valid."""
    import hashlib
    import re
    text = ""
    for name in names:
        p = os.path.join(ROOT, "sliding_window_attention_swa_amd", "csrc", name)
        text += open(p, encoding="utf-8").read() + "\n"
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


PREFILL_SOURCE = ("swa_prefill_bf16.hip", "swa_tile_math.h")
PREFILL_F32_SOURCE = ("swa_prefill_f32.hip", "swa_tile_math.h")
DECODE_SOURCE = ("swa_ring.hip",)


def summarize_pmc(paths):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the calibration copy and
    of the step's kernels -> HBM bytes per launch.  Each counter is scaled by
    (known copy bytes) / (what that counter reads for the copy).  The copy is
    the largest runtime buffer copy (__amd_rocclr_copyBuffer) in the run."""
    import csv
    kinds = {"prefill_bf16_kernel": "prefill", "decode_split_kernel": "decode",
             "decode_combine_kernel": "decode_combine"}
    per = {}  # (kind, counter) -> value
    for path in paths:
        for r in csv.DictReader(open(path)):
            name, ctr, val = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name:
                per[("copy", ctr)] = max(per.get(("copy", ctr), 0.0), val)
                continue
            for pat, kind in kinds.items():
                if pat in name:
                    per[(kind, ctr)] = per.get((kind, ctr), 0.0) + val
    factors = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        copy_kib = per.get(("copy", ctr))
        if not copy_kib:
            print("no calibration copy for %s" % ctr, file=sys.stderr)
            return 1
        factors[ctr] = COPY_BYTES / (copy_kib * 1024.0)
        print("%s: the %d MiB copy reads %.0f KiB -> factor %.4f"
              % (ctr, COPY_BYTES >> 20, copy_kib, factors[ctr]))
    totals = {}
    for kind in ("prefill", "decode", "decode_combine"):
        parts = []
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            kib = per.get((kind, ctr))
            if kib is None:
                continue
            b = kib * 1024.0 * factors[ctr]
            parts.append(b)
            print("%s %s: %.0f KiB -> %.0f bytes" % (kind, ctr, kib, b))
        if len(parts) == 2:
            totals[kind] = int(sum(parts))
    if "prefill" not in totals:
        print("no prefill counters", file=sys.stderr)
        return 1
    print("traffic_bytes_per_launch: %d" % totals["prefill"])
    print("traffic_kernel_sha256: %s" % source_hash(PREFILL_SOURCE))
    if "decode" in totals:
        print("decode_traffic_bytes_per_launch: %d" % totals["decode"])
        print("decode_traffic_kernel_sha256: %s" % source_hash(DECODE_SOURCE))
    return 0


# the HBM-bound prefill configurations whose traffic --pmc-small measures,
# in dispatch order, with the kernel each one runs
SMALL_TRAFFIC = ((2, "prefill_short_kernel"), (5, "prefill_bf16_kernel"))


def pmc_small():
    """Counter workload for the HBM-bound prefill configurations: the
    calibration copy, then TinyMistral and Longformer once each, every one
    after a 1 GiB read that evicts the L2s and the Infinity Cache."""
    import torch
    import sliding_window_attention_swa_amd as swa
    dev = torch.device("cuda:0")
    swa.load()
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)  # read, not written: no dirty lines
    flush_max = torch.empty((), dtype=torch.int32, device=dev)
    for wl, _ in SMALL_TRAFFIC:
        c = si.WORKLOADS[wl]
        q, k, v = (si.to_torch(t, dev) for t in si.prefill_inputs(wl))
        out = torch.empty_like(q)
        torch.amax(flush, dim=0, out=flush_max)
        torch.cuda.synchronize()
        swa.prefill(q, k, v, c["W"], mode=c["mode"], out=out)
        torch.cuda.synchronize()
        del q, k, v, out
    print("pmc small workload done", flush=True)
    return 0


def summarize_pmc_small(paths):
    """HBM bytes of each --pmc-small configuration (counters scaled by the
    calibration copy) against its algorithmic Q + K + V read and O write."""
    import csv
    per, copy = {}, {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            name, ctr, val = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
            if "copyBuffer" in name:
                copy[ctr] = max(copy.get(ctr, 0.0), val)
            for wl, pat in SMALL_TRAFFIC:
                if pat in name:
                    per[(wl, ctr)] = per.get((wl, ctr), 0.0) + val
    for wl, _ in SMALL_TRAFFIC:
        c = si.WORKLOADS[wl]
        rd = 2 * c["T"] * c["d"] * c["B"] * (c["Hq"] + 2 * c["Hkv"])
        wr = 2 * c["T"] * c["d"] * c["B"] * c["Hq"]
        got = {}
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            if ctr in copy and (wl, ctr) in per:
                got[ctr] = per[(wl, ctr)] * COPY_BYTES / copy[ctr]
        print("%s: read %s bytes (algorithmic %d), written %s bytes (algorithmic %d)" % (
            c["name"], "%.0f" % got["FETCH_SIZE"] if "FETCH_SIZE" in got else "-", rd,
            "%.0f" % got["WRITE_SIZE"] if "WRITE_SIZE" in got else "-", wr))
    return 0


def pmc_config(wl, dtype="bf16"):
    """Counter workload of one prefill configuration (its inputs in `dtype`):
    its kernel once after a 1 GiB read that evicts the L2s and the Infinity
    Cache, then once warm."""
    import torch
    import sliding_window_attention_swa_amd as swa
    dev = torch.device("cuda:0")
    swa.load()
    c = si.WORKLOADS[wl]
    q, k, v = (si.to_torch(t, dev) for t in si.prefill_inputs(wl, dtype=dtype))
    out = torch.empty_like(q)
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    flush_max = torch.empty((), dtype=torch.int32, device=dev)
    torch.amax(flush, dim=0, out=flush_max)
    torch.cuda.synchronize()
    for _ in range(2):
        swa.prefill_dilated(q, k, v, c["W"], c.get("dilation", 1), mode=c["mode"], out=out)
        torch.cuda.synchronize()
    print("pmc workload %d (%s, %s) done" % (wl, c["name"], dtype), flush=True)
    return 0


def trace_global(wl, calls=13):
    """Kernel-trace workload of a window-plus-global-tokens configuration:
    `calls` launches of the whole pass (window and global-row launch, then
    the merge), each after a 1 GiB read that evicts the caches."""
    import torch
    import sliding_window_attention_swa_amd as swa
    dev = torch.device("cuda:0")
    swa.load()
    c = si.WORKLOADS[wl]
    q, k, v = (si.to_torch(t, dev) for t in si.prefill_inputs(wl))
    out = torch.empty_like(q)
    gpos = torch.tensor(c["global_pos"], dtype=torch.int32, device=dev)
    ws = swa.global_workspace(c["T"], c["B"] * c["Hq"], len(c["global_pos"]), c["d"], dev)
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    flush_max = torch.empty((), dtype=torch.int32, device=dev)
    for _ in range(calls):
        torch.amax(flush, dim=0, out=flush_max)
        swa.prefill_global(q, k, v, c["W"], gpos, mode=c["mode"], scale=1.0 / math.sqrt(c["d"]),
                           out=out, workspace=ws, dilation=c.get("dilation", 1))
    torch.cuda.synchronize()
    print("trace workload %d (%s) done" % (wl, c["name"]), flush=True)
    return 0


def summarize_config_counters(paths, wl):
    """Per-dispatch SQ / TA counters of a --pmc-config run (the first, flushed
    dispatch of the prefill kernel), with the derived issue and wait figures."""
    import csv
    c = si.WORKLOADS[wl]
    per, dur, first = {}, {}, {}
    for path in paths:  # one pass per file; a counter taken in several passes counts once
        rows = [r for r in csv.DictReader(open(path)) if "prefill_" in r["Kernel_Name"]]
        if not rows:
            continue
        d0 = min(int(r["Dispatch_Id"]) for r in rows)
        mine = {}
        for r in rows:
            if int(r["Dispatch_Id"]) != d0:
                continue
            first[r["Counter_Name"]] = short_kernel_name(r["Kernel_Name"])
            mine[r["Counter_Name"]] = mine.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            dur[r["Counter_Name"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        for k, v in mine.items():
            per.setdefault(k, v)
    if not per:
        print("no prefill dispatch in the counter files", file=sys.stderr)
        return 1
    g = per.get
    kernels = sorted(set(first.values()))
    f32 = any("f32" in kn for kn in kernels)
    print("%s: kernel %s" % (c["name"], kernels))
    print("counters_kernel_sha256: %s" % source_hash(PREFILL_F32_SOURCE if f32 else PREFILL_SOURCE))
    for k in sorted(per):
        print("  %-32s %.6g" % (k, per[k]))
    t = max(dur.values())
    print("  dispatch (under the profiler) %.1f us" % (t * 1e6))
    # cycles of one XCD during the dispatch: GRBM_GUI_ACTIVE sums the 8 XCDs
    # (it also counts the profiler's short window around the dispatch)
    cycles = g("GRBM_GUI_ACTIVE") / N_XCD if g("GRBM_GUI_ACTIVE") else t * CLOCK_MAX_HZ
    print("  cycles per XCD %.0f -> clock %.0f MHz during the dispatch" % (cycles, cycles / t / 1e6))
    if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
        print("  MFMA busy %.1f%% of SIMD cycles"
              % (100.0 * g("SQ_VALU_MFMA_BUSY_CYCLES") / (cycles * N_SIMD)))
    if f32 and g("SQ_INSTS_MFMA"):
        # v_mfma_f32_32x32x2_f32: 4096 FLOP, 64 cycles of a SIMD's matrix core
        # (157.3 TFLOP/s = 1024 SIMDs x 2.4 GHz x 64 FLOP per cycle)
        print("  fp32 matrix products %.4g = %.1f cycles each of the busy count"
              % (g("SQ_INSTS_MFMA"), (g("SQ_VALU_MFMA_BUSY_CYCLES") or 0) / g("SQ_INSTS_MFMA")))
    if g("SQ_LDS_IDX_ACTIVE") is not None:
        print("  LDS busy (indexed access) %.1f%% of CU cycles"
              % (100.0 * g("SQ_LDS_IDX_ACTIVE") / (cycles * N_CU)))
    if g("SQ_LDS_BANK_CONFLICT") is not None:
        print("  LDS bank-conflict cycles %.3g" % g("SQ_LDS_BANK_CONFLICT"))
    if g("SQ_WAVE_CYCLES"):
        wc = g("SQ_WAVE_CYCLES")
        for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_SCA"):
            if g(k) is not None:
                print("  %-22s %.1f%% of wave cycles" % (k, 100.0 * g(k) / wc))
        if g("SQ_WAVES"):
            print("  waves %d, average life %.0f cycles" % (g("SQ_WAVES"), wc / g("SQ_WAVES")))
    if g("SQ_INSTS_VALU") and g("SQ_INSTS_MFMA"):
        print("  VALU instructions per MFMA %.2f" % (g("SQ_INSTS_VALU") / g("SQ_INSTS_MFMA")))
    if g("SQ_INSTS_VALU_TRANS_F32"):
        exps = band_pairs(c["T"], c["W"], c["mode"], c.get("dilation", 1)) * c["Hq"] * c["B"] / 64.0
        print("  transcendental instructions %.4g = %.3f x one exp per in-window score"
              % (g("SQ_INSTS_VALU_TRANS_F32"), g("SQ_INSTS_VALU_TRANS_F32") / exps))
    if g("SQ_LEVEL_WAVES") and g("SQ_BUSY_CYCLES"):
        print("  waves resident on average %.0f" % (g("SQ_LEVEL_WAVES") / g("SQ_BUSY_CYCLES")))
    return 0


def _short_mangled(name):
    """name<args> of a mangled kernel of this library: nested length-prefixed
    identifiers, then template arguments that are integers (Li128E) or the
    element types bf16 (DF16b) and float (f)."""
    import re
    i, parts = 3, []
    while i < len(name) and name[i].isdigit():
        n = re.match(r"\d+", name[i:]).group(0)
        i += len(n)
        parts.append(name[i:i + int(n)])
        i += int(n)
    if not parts:
        return None
    args = []
    if name[i:i + 1] == "I":
        i += 1
        while i < len(name) and name[i] != "E":
            m = re.match(r"L[a-z](-?\d+)E|(DF16b)|([fb])", name[i:])
            if not m:
                return None
            args.append(m.group(1) or {"DF16b": "bf16", "f": "float", "b": "bool"}[m.group(2) or m.group(3)])
            i += len(m.group(0))
    return parts[-1] + ("<%s>" % ", ".join(args) if args else "")


def short_kernel_name(name):
    """A kernel's name without namespaces, return type and parameter list
    (demangled first when the trace left it mangled)."""
    if name.startswith("_ZN"):
        name = _short_mangled(name) or name
    name = name.replace("(anonymous namespace)::", "")
    name = name.split("(")[0]
    if name.startswith("void "):
        name = name[5:]
    return name.replace("swa::", "").replace("at::native::", "")


def summarize_kernel_trace(paths, skip):
    """Per-kernel durations from a rocprofv3 --kernel-trace CSV of a benchmark
    run, without the first `skip` dispatches of each kernel (the untimed
    warm-up steps): the calls the timed region made."""
    import csv
    calls = {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            name = short_kernel_name(r["Kernel_Name"])
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            calls.setdefault(name, []).append((t0, (t1 - t0) * 1e-3))
    rows = []
    for name, cs in calls.items():
        cs.sort()
        us = [u for _, u in cs[skip:]]
        if us:
            rows.append((sum(us), name, len(us), sum(us) / len(us), min(us), max(us)))
    if not rows:
        print("no kernel dispatches after the warm-ups", file=sys.stderr)
        return 1
    total = sum(r[0] for r in rows)
    print("| kernel | calls | average (us) | min (us) | max (us) | share |")
    print("|---|---|---|---|---|---|")
    for tot, name, n, avg, lo, hi in sorted(rows, reverse=True):
        print("| %s | %d | %.1f | %.1f | %.1f | %.1f%% |" % (name, n, avg, lo, hi, 100.0 * tot / total))
    return 0


N_XCD, N_CU, N_SIMD = 8, 256, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs
CLOCK_MAX_HZ = 2.4e9  # MI355X's peak engine clock
MFMA_FLOP_PER_SIMD_CYCLE = 1024  # v_mfma_f32_32x32x16_bf16: 32768 FLOP in 32 cycles


def summarize_counters(paths):
    """MFMA and instruction-mix figures of the prefill (and decode) dispatch
    of a --pmc-workload run, from rocprofv3 counter CSVs: each counter is
    summed over the dispatch's hardware instances (GRBM_GUI_ACTIVE over the
    8 XCDs, SQ counters over SEs and SIMDs)."""
    import csv
    kinds = {"prefill_bf16_kernel": "prefill", "decode_split_kernel": "decode"}
    per, dur = {}, {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            for pat, kind in kinds.items():
                if pat in r["Kernel_Name"]:
                    per[(kind, r["Counter_Name"])] = per.get((kind, r["Counter_Name"]), 0.0) + \
                        float(r["Counter_Value"])
                    dur[kind] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    if "prefill" not in dur:
        print("no prefill dispatch in the counter files", file=sys.stderr)
        return 1
    print("counters_kernel_sha256: %s" % source_hash(PREFILL_SOURCE))
    for kind in ("prefill", "decode"):
        if kind not in dur:
            continue
        g = lambda c: per.get((kind, c))  # noqa: E731
        print("%s: dispatch %.1f us" % (kind, dur[kind] * 1e6))
        for c in sorted(k for (kk, k) in per if kk == kind):
            print("  %-30s %.6g" % (c, per[(kind, c)]))
        gui = g("GRBM_GUI_ACTIVE")
        if not gui:
            continue
        cycles = gui / N_XCD
        clock = cycles / dur[kind]
        print("  cycles per XCD %.0f -> clock %.0f MHz during the dispatch" % (cycles, clock / 1e6))
        busy = g("SQ_VALU_MFMA_BUSY_CYCLES")
        if busy is not None:
            print("  MFMA busy: %.1f%% of SIMD cycles" % (100.0 * busy / (cycles * N_SIMD)))
        mops = g("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        if mops is not None and kind == "prefill":
            flops, _ = prefill_work()
            issued = mops * 512
            print("  MFMA FLOPs issued %.4g = %.3f x the in-window FLOPs" % (issued, issued / flops))
            print("  issued MFMA rate %.0f TFLOP/s; peak at this clock %.0f TFLOP/s (%.1f%%); "
                  "in-window rate %.0f TFLOP/s" % (
                      issued / dur[kind] / 1e12, N_SIMD * MFMA_FLOP_PER_SIMD_CYCLE * clock / 1e12,
                      100.0 * issued / dur[kind] / (N_SIMD * MFMA_FLOP_PER_SIMD_CYCLE * clock),
                      flops / dur[kind] / 1e12))
        if g("SQ_INSTS_VALU") and g("SQ_INSTS_MFMA"):
            print("  VALU instructions per MFMA: %.2f" % (g("SQ_INSTS_VALU") / g("SQ_INSTS_MFMA")))
        if g("SQ_INSTS_VALU_TRANS_F32") and kind == "prefill":
            c = si.WORKLOADS[3]
            exps = band_pairs_causal(c["T"], c["W"]) * c["Hq"] * c["B"] / 64.0
            print("  transcendental instructions %.4g = %.3f x one exp per in-window score"
                  % (g("SQ_INSTS_VALU_TRANS_F32"), g("SQ_INSTS_VALU_TRANS_F32") / exps))
        if g("SQ_LDS_BANK_CONFLICT") is not None:
            print("  LDS bank-conflict cycles: %.3g (%.2f%% of SIMD cycles)"
                  % (g("SQ_LDS_BANK_CONFLICT"), 100.0 * g("SQ_LDS_BANK_CONFLICT") / (cycles * N_SIMD)))
        if g("SQ_LDS_IDX_ACTIVE") is not None:
            print("  LDS busy (indexed access): %.1f%% of CU cycles"
                  % (100.0 * g("SQ_LDS_IDX_ACTIVE") / (cycles * N_CU)))
        if g("SQ_INSTS_LDS_LOAD_BANDWIDTH") is not None:
            nbytes = 64.0 * g("SQ_INSTS_LDS_LOAD_BANDWIDTH")
            print("  LDS bytes read %.4g = %.1f B per CU cycle" % (nbytes, nbytes / (cycles * N_CU)))
    return 0


def cpu_baseline(pos_np, q_dec, kr, vr, qkv_pre):
    """fp64 oracle on the host cores over a bounded sample of one step (about
    15 s on 16 cores): all 32 prefill query heads (all 16384 rows each) and 32
    of the 64 decode sequences (all 32 heads).  Reported as in-window
    TFLOP/s."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = len(os.sched_getaffinity(0))
    c3, c4 = si.WORKLOADS[3], si.WORKLOADS[4]
    q, k, v = qkv_pre
    heads = [(0, h) for h in range(c3["Hq"])]
    t0 = time.perf_counter()
    oracle.attention_banded(q.values, k.values, v.values, c3["W"], c3["mode"],
                            1 / math.sqrt(c3["d"]), heads=heads)
    t1 = time.perf_counter()
    nb = 32
    oracle.decode(q_dec.values[:nb], kr.values[:nb], vr.values[:nb], pos_np[:nb],
                  1 / math.sqrt(c4["d"]))
    t2 = time.perf_counter()
    pre_flops = 4 * c3["d"] * band_pairs_causal(c3["T"], c3["W"]) * len(heads)
    dec_rows = int(np.minimum(pos_np[:nb].astype(np.int64) + 1, c4["W"]).sum())
    dec_flops = 4 * c4["d"] * dec_rows * c4["Hq"]
    secs = t2 - t0
    return {
        "value": (pre_flops + dec_flops) / secs / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": "fp64 numpy oracle: prefill of %d of 32 query heads (T=16384, W=4096, "
                  "d=128, every row; %.1f s) + decode of %d of 64 sequences (32 heads, W=4096; "
                  "%.1f s)" % (len(heads), t1 - t0, nb, t2 - t1),
        "seconds": secs,
    }


def cpu_oracle_configs():
    """The fp64 oracle's own speed on the host cores, per configuration: the
    banded form on a bounded sample of heads (every row of each) for the
    prefill configurations and a sample of sequences for the decode, with all
    BLAS threads and with one.  One JSON line per (configuration, threads)."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    all_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    samples = []
    for wl, heads in ((2, 32), (5, 8), (3, 2)):
        c = si.WORKLOADS[wl]
        q, k, v = si.prefill_inputs(wl)
        hs = [(b, h) for b in range(c["B"]) for h in range(c["Hq"])][:heads]
        flops = 4 * c["d"] * band_pairs(c["T"], c["W"], c["mode"]) * len(hs)
        fn = (lambda q=q, k=k, v=v, c=c, hs=hs: oracle.attention_banded(
            q.values, k.values, v.values, c["W"], c["mode"], 1 / math.sqrt(c["d"]), heads=hs))
        samples.append((c["name"], "%d of %d heads, every row" % (len(hs), c["B"] * c["Hq"]),
                        flops, fn))
    c4 = si.WORKLOADS[4]
    qd, kr, vr, pos = si.decode_inputs(4)
    nb = 8
    rows = int(np.minimum(pos[:nb].astype(np.int64) + 1, c4["W"]).sum())
    samples.append((c4["name"], "%d of %d sequences" % (nb, c4["B"]), 4 * c4["d"] * rows * c4["Hq"],
                    lambda: oracle.decode(qd.values[:nb], kr.values[:nb], vr.values[:nb], pos[:nb],
                                          1 / math.sqrt(c4["d"]))))
    for name, what, flops, fn in samples:
        for threads in (all_threads, 1):
            with threadpool_limits(limits=threads):
                t0 = time.perf_counter()
                fn()
                secs = time.perf_counter() - t0
            print(json.dumps({"config": name, "kind": "oracle", "sample": what, "threads": threads,
                              "seconds": round(secs, 3), "gflops": round(flops / secs / 1e9, 2)}),
                  flush=True)
    return 0


def band_pairs(T, W, mode, dilation=1):
    """(query, key) pairs inside the windows of one head, either mode; with a
    dilation, row i has the window's offsets m with i - m * dilation in
    [0, T)."""
    i = np.arange(T, dtype=np.int64)
    if mode == 0:
        if dilation == 1:
            return band_pairs_causal(T, W)
        return int(np.minimum(W - 1, i // dilation).sum() + T)
    h = W // 2
    left = np.minimum(h, i // dilation)
    right = np.minimum(h, (T - 1 - i) // dilation)
    return int((left + right + 1).sum())


def global_pairs(T, W, mode, gpos, dilation=1):
    """(query, key) pairs of one head for the (dilated) window plus global
    tokens: each row's window, plus the global keys outside it (not after the
    row when causal); a global row has every key (every earlier key when
    causal)."""
    i = np.arange(T, dtype=np.int64)
    mlo, mhi = (0, W - 1) if mode == 0 else (-(W // 2), W // 2)  # offsets m = (i - j) / dilation
    top = np.minimum(mhi, i // dilation)                 # keys j = i - m * dilation >= 0
    bot = np.maximum(mlo, -((T - 1 - i) // dilation))    # keys j < T
    n = np.maximum(0, top - bot + 1)
    g = np.asarray(sorted(set(int(x) for x in gpos)), dtype=np.int64)
    diff = i[:, None] - g[None, :]
    m = diff // dilation
    outside = ~((diff % dilation == 0) & (m >= mlo) & (m <= mhi))
    if mode == 0:
        outside &= g[None, :] <= i[:, None]
    n = n + outside.sum(axis=1)
    n[g] = g + 1 if mode == 0 else T
    return int(n.sum())


def measured_peaks(swa, dev, timed):
    """What this GPU sustains (the library's calibration kernels): bf16 matrix
    TFLOP/s of an MFMA loop on N(0,1) operands (the attention inputs'
    distribution), and GB/s of a non-temporal streaming read of 2 GiB (past
    the Infinity Cache); each the best of three grids."""
    import torch
    ops = si.to_torch(si.normal(99, (32768,), "bf16"), dev)
    # grids of whole rounds (three waves per SIMD fit: 768 workgroups fill the
    # chip once) and a long one, at equal FLOPs; the best is the sustained rate
    mfma_tflops = 0.0
    for n_wg in (768, 1536, 6144):
        iters = 1638400 // n_wg
        sink = torch.empty(n_wg * 256, dtype=torch.float32, device=dev)
        flops = n_wg * 4 * iters * 16 * 32768
        ms = timed(lambda: swa.calib_mfma(ops, sink, n_wg, iters), False)
        mfma_tflops = max(mfma_tflops, flops / ms / 1e9)
    src = torch.ones(1 << 29, dtype=torch.int32, device=dev)  # 2 GiB
    best = 0.0
    for grid in (2048, 4096, 8192):
        rsink = torch.empty(grid * 256, dtype=torch.int32, device=dev)
        ms = timed(lambda: swa.calib_stream_read(src, rsink, grid), False)
        best = max(best, src.numel() * 4 / ms / 1e6)
    del src
    # the vector ALU: fp32 FMA and v_exp_f32 chains at eight waves per SIMD;
    # ns per wave instruction per SIMD, and the exponential's cost in FMAs
    vsink = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    ns_per = {}
    for op in (0, 1):
        iters = 8000
        n_instr = swa.calib_vector(op, vsink, 2048, iters)
        ms = timed(lambda: swa.calib_vector(op, vsink, 2048, iters), False)
        ns_per[op] = ms * 1e6 / (n_instr / N_SIMD)
    return {"config": "measured peaks", "mfma_bf16_tflops": round(mfma_tflops, 1),
            "frac_of_published_mfma": round(mfma_tflops / PEAK_BF16_TFLOPS, 3),
            "stream_read_gbs": round(best, 1),
            "frac_of_published_hbm": round(best / PEAK_HBM_GBS, 3),
            "fma_f32_ns_per_wave_instr": round(ns_per[0], 3),
            "exp_f32_ns_per_wave_instr": round(ns_per[1], 3),
            "exp_cost_in_fmas": round(ns_per[1] / ns_per[0], 2),
            "fma_f32_tflops": round(2 * 64 * N_SIMD / ns_per[0] / 1e3, 1)}


def all_configs(reps, peaks_only=False):
    """Every configuration's kernel time, cache-warm (same inputs every
    repetition) and flushed (a 1 GiB read between repetitions evicts the L2s
    and the Infinity Cache), against its binding roofline.  One JSON line per
    configuration."""
    import torch
    import sliding_window_attention_swa_amd as swa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    swa.load()
    # the flush reads 1 GiB with ordinary (cache-allocating) loads: it evicts
    # the L2s and the Infinity Cache without leaving dirty lines whose
    # write-back the timed kernel would pay for
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB
    flush_max = torch.empty((), dtype=torch.int32, device=dev)

    def timed(fn, flushed):
        # every repetition is enqueued before the one host synchronisation, so
        # the device never idles between them; events bracket the kernel alone
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps + 10)]
        for r, (a, b) in enumerate(ev):
            if flushed:
                torch.amax(flush, dim=0, out=flush_max)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev[10:]]))

    peaks = measured_peaks(swa, dev, timed)
    print(json.dumps(peaks), flush=True)
    if peaks_only:
        return 0

    def meas(flops, bytes_, ms):
        """Fraction of the roofline built from the measured peaks."""
        t = max(flops / (peaks["mfma_bf16_tflops"] * 1e12), bytes_ / (peaks["stream_read_gbs"] * 1e9))
        return round(t * 1e3 / ms, 3)

    for wl in (2, 3, 5, 7):
        c = si.WORKLOADS[wl]
        q, k, v = (si.to_torch(t, dev) for t in si.prefill_inputs(wl))
        out = torch.empty_like(q)
        scale = 1.0 / math.sqrt(c["d"])
        dil = c.get("dilation", 1)
        fn = lambda: swa.prefill_dilated(q, k, v, c["W"], dil, mode=c["mode"], scale=scale,  # noqa: E731
                                         out=out)
        flops = 4 * c["d"] * band_pairs(c["T"], c["W"], c["mode"], dil) * c["Hq"] * c["B"]
        bytes_ = 2 * c["T"] * c["d"] * c["B"] * (2 * c["Hq"] + 2 * c["Hkv"])
        t_roof = max(flops / (PEAK_BF16_TFLOPS * 1e12), bytes_ / (PEAK_HBM_GBS * 1e9)) * 1e3
        bound = "mfma" if flops / PEAK_BF16_TFLOPS / 1e12 >= bytes_ / PEAK_HBM_GBS / 1e9 else "hbm"
        row = {"config": c["name"], "kernel": "prefill", "bound": bound,
               "roofline_ms": round(t_roof, 5)}
        for tag, fl in (("warm", False), ("flushed", True)):
            ms = timed(fn, fl)
            row[tag] = {"ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 1),
                        "gbs": round(bytes_ / ms / 1e6, 1), "frac_roofline": round(t_roof / ms, 3),
                        "frac_measured": meas(flops, bytes_, ms)}
        print(json.dumps(row), flush=True)
        del q, k, v, out

    # window (plain, then dilated) plus global tokens
    for wl in (8, 9):
        c = si.WORKLOADS[wl]
        dil = c.get("dilation", 1)
        q, k, v = (si.to_torch(t, dev) for t in si.prefill_inputs(wl))
        out = torch.empty_like(q)
        gpos = torch.tensor(c["global_pos"], dtype=torch.int32, device=dev)
        ws = swa.global_workspace(c["T"], c["B"] * c["Hq"], len(c["global_pos"]), c["d"], dev)
        fn = lambda: swa.prefill_global(q, k, v, c["W"], gpos, mode=c["mode"],  # noqa: E731
                                        scale=1.0 / math.sqrt(c["d"]), out=out, workspace=ws,
                                        dilation=dil)
        flops = (4 * c["d"] * global_pairs(c["T"], c["W"], c["mode"], c["global_pos"], dil)
                 * c["Hq"] * c["B"])
        bytes_ = 2 * c["T"] * c["d"] * c["B"] * (2 * c["Hq"] + 2 * c["Hkv"])
        t_roof = max(flops / (PEAK_BF16_TFLOPS * 1e12), bytes_ / (PEAK_HBM_GBS * 1e9)) * 1e3
        bound = "mfma" if flops / PEAK_BF16_TFLOPS / 1e12 >= bytes_ / PEAK_HBM_GBS / 1e9 else "hbm"
        row = {"config": c["name"], "kernel": "prefill_global", "bound": bound,
               "roofline_ms": round(t_roof, 5)}
        for tag, fl in (("warm", False), ("flushed", True)):
            ms = timed(fn, fl)
            row[tag] = {"ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 1),
                        "gbs": round(bytes_ / ms / 1e6, 1), "frac_roofline": round(t_roof / ms, 3),
                        "frac_measured": meas(flops, bytes_, ms)}
        print(json.dumps(row), flush=True)
        del q, k, v, out, ws

    c = si.WORKLOADS[4]
    q_np, kr_np, vr_np, pos_np = si.decode_inputs(4)
    q, kr, vr = (si.to_torch(t, dev) for t in (q_np, kr_np, vr_np))
    pos = torch.from_numpy(pos_np).to(dev)
    out = torch.empty_like(q)
    ws = swa.decode_workspace(c["B"], c["Hq"], c["W"], c["d"], dev)
    fn = lambda: swa.decode(q, kr, vr, pos, scale=1.0 / math.sqrt(c["d"]), out=out, workspace=ws)  # noqa: E731
    _, kv_bytes, qo_bytes = decode_work(pos_np)
    t_roof = (kv_bytes + qo_bytes) / (PEAK_HBM_GBS * 1e9) * 1e3
    row = {"config": c["name"], "kernel": "decode", "bound": "hbm", "roofline_ms": round(t_roof, 5)}
    for tag, fl in (("warm", False), ("flushed", True)):
        ms = timed(fn, fl)
        row[tag] = {"ms": round(ms, 5), "kv_gbs": round(kv_bytes / ms / 1e6, 1),
                    "frac_roofline": round(t_roof / ms, 3),
                    "frac_measured": meas(0, kv_bytes + qo_bytes, ms)}
    print(json.dumps(row), flush=True)
    del out, ws

    # the same decode with 4 attention sinks beside each ring
    ks = si.to_torch(si.normal(si.seed_for(4, si.ROLE_K_RING), (c["B"], c["Hkv"], 4, c["d"]), c["dtype"]), dev)
    vs = si.to_torch(si.normal(si.seed_for(4, si.ROLE_V_RING), (c["B"], c["Hkv"], 4, c["d"]), c["dtype"]), dev)
    out = torch.empty_like(q)
    ws = swa.decode_sinks_workspace(c["B"], c["Hq"], c["W"], c["d"], dev)
    fn = lambda: swa.decode_sinks(q, kr, vr, ks, vs, pos, scale=1.0 / math.sqrt(c["d"]), out=out,  # noqa: E731
                                  workspace=ws)
    row = {"config": c["name"] + " + 4 sinks", "kernel": "decode_sinks", "bound": "hbm",
           "roofline_ms": round(t_roof, 5)}
    for tag, fl in (("warm", False), ("flushed", True)):
        ms = timed(fn, fl)
        row[tag] = {"ms": round(ms, 5), "kv_gbs": round(kv_bytes / ms / 1e6, 1),
                    "frac_roofline": round(t_roof / ms, 3),
                    "frac_measured": meas(0, kv_bytes + qo_bytes, ms)}
    print(json.dumps(row), flush=True)
    del q, kr, vr, ks, vs, out, ws

    # chunked prefill into full rings, then the chunk's append
    c = si.WORKLOADS[6]
    tensors = si.chunk_inputs(6)
    q, k, v, kr, vr = (si.to_torch(t, dev) for t in tensors[:5])
    pos_np = tensors[5]
    pos = torch.from_numpy(pos_np).to(dev)
    out = torch.empty_like(q)
    fn = lambda: swa.prefill_chunk(q, k, v, kr, vr, pos, scale=1.0 / math.sqrt(c["d"]), out=out)  # noqa: E731
    flops, bytes_ = chunk_work(c, pos_np)
    t_roof = max(flops / (PEAK_BF16_TFLOPS * 1e12), bytes_ / (PEAK_HBM_GBS * 1e9)) * 1e3
    bound = "mfma" if flops / PEAK_BF16_TFLOPS / 1e12 >= bytes_ / PEAK_HBM_GBS / 1e9 else "hbm"
    row = {"config": c["name"], "kernel": "prefill_chunk", "bound": bound,
           "roofline_ms": round(t_roof, 5)}
    for tag, fl in (("warm", False), ("flushed", True)):
        ms = timed(fn, fl)
        row[tag] = {"ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 1),
                    "gbs": round(bytes_ / ms / 1e6, 1), "frac_roofline": round(t_roof / ms, 3),
                    "frac_measured": meas(flops, bytes_, ms)}
    print(json.dumps(row), flush=True)
    # the append rewrites the same slots every repetition (same positions)
    fn = lambda: swa.cache_append_chunk(kr, vr, pos, k, v)  # noqa: E731
    rows = c["B"] * c["Hkv"] * min(c["n"], c["W"])
    bytes_ = 2 * rows * c["d"] * 2 * 2  # K and V rows, read once and written once
    t_roof = bytes_ / (PEAK_HBM_GBS * 1e9) * 1e3
    row = {"config": c["name"] + " append", "kernel": "append_chunk", "bound": "hbm",
           "roofline_ms": round(t_roof, 5)}
    for tag, fl in (("warm", False), ("flushed", True)):
        ms = timed(fn, fl)
        row[tag] = {"ms": round(ms, 5), "gbs": round(bytes_ / ms / 1e6, 1),
                    "frac_roofline": round(t_roof / ms, 3),
                    "frac_measured": meas(0, bytes_, ms)}
    print(json.dumps(row), flush=True)
    del q, k, v, kr, vr, out

    # fp32 inputs (no named configuration is fp32 beyond the 16-token toy):
    # the Mistral-7B and Longformer prefills and the Mistral-7B chunk in fp32,
    # against the fp32 matrix-core roofline (4-byte elements)
    def fp32_row(name, kernel, flops, bytes_, fn):
        t_roof = max(flops / (PEAK_FP32_MFMA_TFLOPS * 1e12), bytes_ / (PEAK_HBM_GBS * 1e9)) * 1e3
        bound = "mfma" if flops / PEAK_FP32_MFMA_TFLOPS / 1e12 >= bytes_ / PEAK_HBM_GBS / 1e9 else "hbm"
        row = {"config": name, "kernel": kernel, "bound": bound, "roofline_ms": round(t_roof, 5),
               "peak_tflops": PEAK_FP32_MFMA_TFLOPS}
        for tag, fl in (("warm", False), ("flushed", True)):
            ms = timed(fn, fl)
            row[tag] = {"ms": round(ms, 5), "tflops": round(flops / ms / 1e9, 1),
                        "gbs": round(bytes_ / ms / 1e6, 1), "frac_roofline": round(t_roof / ms, 3)}
        print(json.dumps(row), flush=True)

    for wl in (3, 5):
        c = si.WORKLOADS[wl]
        q, k, v = (si.to_torch(t, dev) for t in si.prefill_inputs(wl, dtype="f32"))
        out = torch.empty_like(q)
        fn = lambda: swa.prefill(q, k, v, c["W"], mode=c["mode"], scale=1.0 / math.sqrt(c["d"]),  # noqa: E731
                                 out=out)
        flops = 4 * c["d"] * band_pairs(c["T"], c["W"], c["mode"], 1) * c["Hq"] * c["B"]
        bytes_ = 4 * c["T"] * c["d"] * c["B"] * (2 * c["Hq"] + 2 * c["Hkv"])
        fp32_row(c["name"] + " in fp32", "prefill_f32", flops, bytes_, fn)
        del q, k, v, out
    c = si.WORKLOADS[6]
    tensors = si.chunk_inputs(6, dtype="f32")
    q, k, v, kr, vr = (si.to_torch(t, dev) for t in tensors[:5])
    pos = torch.from_numpy(tensors[5]).to(dev)
    out = torch.empty_like(q)
    fn = lambda: swa.prefill_chunk(q, k, v, kr, vr, pos, scale=1.0 / math.sqrt(c["d"]), out=out)  # noqa: E731
    flops, bytes_ = chunk_work(c, tensors[5])
    fp32_row(c["name"] + " in fp32", "prefill_chunk_f32", flops, 2 * bytes_, fn)
    return 0


def chunk_work(c, pos):
    """In-window FLOPs and algorithmic bytes of a chunked prefill: row i of a
    chunk at position p sees min(p + i + 1, W) keys; the bytes are Q, O, the
    chunk's K and V, and the ring rows some window reads (min(p, W - 1) per
    KV head, K and V), bf16."""
    n, W, d = c["n"], c["W"], c["d"]
    i = np.arange(n, dtype=np.int64)
    keys = sum(int(np.minimum(int(p) + i + 1, W).sum()) for p in pos if p >= 0)
    flops = 4 * d * keys * c["Hq"]
    ring_rows = sum(min(int(p), W - 1) for p in pos if p >= 0)
    bytes_ = 2 * d * (c["B"] * n * (2 * c["Hq"] + 2 * c["Hkv"]) + 2 * c["Hkv"] * ring_rows)
    return flops, bytes_


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="run one plain copy of %d MiB, then one step, for counter collection"
                    % (COPY_BYTES >> 20))
    ap.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs of a "
                         "--pmc-workload run into the prefill traffic summary")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="turn rocprofv3 MFMA / instruction counter CSVs of a --pmc-workload run "
                         "into utilisation figures")
    ap.add_argument("--cpu-oracle", action="store_true",
                    help="instead of the benchmark line: the fp64 oracle's speed per "
                         "configuration on the host cores, all threads and one")
    ap.add_argument("--pmc-small", action="store_true",
                    help="instead of the benchmark line: the counter workload of the HBM-bound "
                         "prefill configurations (run under rocprofv3 --pmc)")
    ap.add_argument("--summarize-pmc-small", nargs="+", metavar="CSV",
                    help="HBM bytes of the --pmc-small configurations from FETCH_SIZE / "
                         "WRITE_SIZE counter CSVs")
    ap.add_argument("--pmc-config", type=int, metavar="N",
                    help="instead of the benchmark line: the counter workload of prefill "
                         "configuration N (run under rocprofv3 --pmc)")
    ap.add_argument("--summarize-config-counters", nargs="+", metavar="CSV",
                    help="SQ counters of a --pmc-config run (with --config N)")
    ap.add_argument("--config", type=int, default=5, help="configuration of the summary")
    ap.add_argument("--pmc-dtype", choices=("bf16", "f32"), default="bf16",
                    help="input type of the --pmc-config workload")
    ap.add_argument("--trace-global", type=int, metavar="N",
                    help="instead of the benchmark line: 13 flushed calls of the window plus "
                         "global tokens configuration N (run under rocprofv3 --kernel-trace)")
    ap.add_argument("--summarize-kernel-trace", nargs="+", metavar="CSV",
                    help="per-kernel times of a rocprofv3 --kernel-trace run of the benchmark "
                         "line, without the --warmup steps' dispatches")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measurement of this GPU's sustained matrix and read rates "
                         "after the timed steps")
    ap.add_argument("--peaks", action="store_true",
                    help="instead of the benchmark line: the matrix-core and streaming-read "
                         "rates this GPU sustains (the library's calibration kernels)")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the benchmark line: every configuration, cache-warm and "
                         "flushed, against its roofline (one JSON line each)")
    args = ap.parse_args()
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.summarize_pmc_small:
        return summarize_pmc_small(args.summarize_pmc_small)
    if args.pmc_small:
        return pmc_small()
    if args.pmc_config:
        return pmc_config(args.pmc_config, args.pmc_dtype)
    if args.summarize_config_counters:
        return summarize_config_counters(args.summarize_config_counters, args.config)
    if args.trace_global:
        return trace_global(args.trace_global)
    if args.summarize_kernel_trace:
        return summarize_kernel_trace(args.summarize_kernel_trace, args.warmup)
    if args.cpu_oracle:
        return cpu_oracle_configs()
    if args.all_configs or args.peaks:
        return all_configs(max(args.steps, 50), peaks_only=args.peaks)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the sliding-window attention path here is a "
              "single-device library (heads and sequences shard without communication); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import sliding_window_attention_swa_amd as swa

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    swa.load()
    c3, c4 = si.WORKLOADS[3], si.WORKLOADS[4]

    # ---- inputs, resident in HBM before timing
    qkv_pre = si.prefill_inputs(3)
    q_pre, k_pre, v_pre = (si.to_torch(t, dev) for t in qkv_pre)
    out_pre = torch.empty_like(q_pre)
    q_dec_np, kr_np, vr_np, pos_np = si.decode_inputs(4)
    q_dec = si.to_torch(q_dec_np, dev)
    k_ring = si.to_torch(kr_np, dev)
    v_ring = si.to_torch(vr_np, dev)
    pos = torch.from_numpy(pos_np).to(dev)
    new_k = si.to_torch(si.normal(si.seed_for(4, 4), (c4["B"], c4["Hkv"], c4["d"]), si.BF16), dev)
    new_v = si.to_torch(si.normal(si.seed_for(4, 5), (c4["B"], c4["Hkv"], c4["d"]), si.BF16), dev)
    out_dec = torch.empty_like(q_dec)
    ws = swa.decode_workspace(c4["B"], c4["Hq"], c4["W"], c4["d"], dev)
    s_pre = 1.0 / math.sqrt(c3["d"])
    s_dec = 1.0 / math.sqrt(c4["d"])

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        swa.prefill(q_pre, k_pre, v_pre, c3["W"], mode=c3["mode"], scale=s_pre, out=out_pre)
        if ev is not None:
            ev[1].record()
        swa.cache_append(k_ring, v_ring, pos, new_k, new_v)
        if ev is not None:
            ev[2].record()
        swa.decode(q_dec, k_ring, v_ring, pos, scale=s_dec, out=out_dec, workspace=ws)
        if ev is not None:
            ev[3].record()

    if args.pmc_workload:
        # a plain copy kernel of known size calibrates the byte counters
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        print("pmc workload done", flush=True)
        return 0

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(events[i])
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms_step = start.elapsed_time(stop) / args.steps
    ms_pre = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    ms_app = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    ms_dec = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))

    pre_flops, pre_bytes = prefill_work()
    dec_flops, dec_kv_bytes, dec_qo_bytes = decode_work(pos_np)
    step_flops = pre_flops + dec_flops
    value = step_flops / (ms_step * 1e-3) / 1e12
    pre_tflops = pre_flops / (ms_pre * 1e-3) / 1e12
    dec_gbs = dec_kv_bytes / (ms_dec * 1e-3) / 1e9

    traffic = read_traffic("", PREFILL_SOURCE)
    dec_traffic = read_traffic("decode_", DECODE_SOURCE)
    peaks = None
    if not args.no_peaks:  # after the timed region: what this GPU sustains
        def timed(fn, flushed):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(8)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            return float(np.median([a.elapsed_time(b) for a, b in ev[2:]]))
        peaks = measured_peaks(swa, dev, timed)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) rounded to bf16, resident in HBM",
        "config": {
            "workload": "Mistral-7B-shaped SWA step: causal prefill B=1 T=16384 W=4096 "
                        "Hq/Hkv=32/8 d=128 + ring append + split-K ring decode B=64 "
                        "W=4096 Hq/Hkv=32/8 d=128 pos~U[4096,32768)",
            "prefill": {"B": c3["B"], "T": c3["T"], "W": c3["W"], "Hq": c3["Hq"],
                        "Hkv": c3["Hkv"], "d": c3["d"], "mode": "causal"},
            "decode": {"B": c4["B"], "W": c4["W"], "Hq": c4["Hq"], "Hkv": c4["Hkv"],
                       "d": c4["d"], "pos": [int(c4["pos_lo"]), int(c4["pos_hi"])]},
        },
        "parts": {
            "prefill": {"ms": round(ms_pre, 4), "in_window_tflops": round(pre_tflops, 2),
                        "frac_bf16_peak": round(pre_tflops / PEAK_BF16_TFLOPS, 4)},
            "append": {"ms": round(ms_app, 4)},
            "decode": {"ms": round(ms_dec, 4), "kv_read_gbs": round(dec_gbs, 1),
                       "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4),
                       "kv_bytes": dec_kv_bytes},
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(pre_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "prefill_bf16_kernel<128, causal>",
            "algorithmic_flops_per_launch": pre_flops,
            "algorithmic_bytes_per_launch": pre_bytes,
            "measured_peak": peaks["mfma_bf16_tflops"] if peaks else None,
            "frac_measured": round(pre_tflops / peaks["mfma_bf16_tflops"], 4) if peaks else None,
        },
        "decode_roofline": {
            "bound": "hbm",
            "achieved": round(dec_gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(dec_gbs / PEAK_HBM_GBS, 4),
            "traffic": dec_traffic,
            "kernel": "decode_split_kernel<bf16, 128, 4>",
            "algorithmic_bytes_per_launch": dec_kv_bytes + dec_qo_bytes,
            "measured_peak": peaks["stream_read_gbs"] if peaks else None,
            "frac_measured": round(dec_gbs / peaks["stream_read_gbs"], 4) if peaks else None,
        },
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pos_np, q_dec_np, kr_np, vr_np, qkv_pre)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
