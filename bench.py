#!/usr/bin/env python3
"""Throughput of exact tiled attention, forward + backward, on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
fa_fwd (O, LSE), then the backward's three stages fa_bwd_preprocess,
fa_bwd_dkdv and fa_bwd_dq (together exactly fa_bwd).  Inputs are resident
in HBM before the timed region; W warm-up steps, then K timed steps between
two device synchronisations.  HIP events recorded on the launch stream around
every kernel give each kernel's average duration over the same timed steps.

value = credited FLOPs of a step / step time, with the credited counts
fwd = 4*B*H*N^2*d and bwd = 10*B*H*N^2*d, both halved for a causal mask.
``target`` holds the backward's own credited rate over the dense bf16 peak
beside the 0.40 bar the backward is built against.  The backward's dQ method
is the library's choice for the workspace given (the dS hand-off; with
FA_DQ_MODE=recompute the recomputing dQ kernel), reported as detail.dq_mode.

Prints one JSON line.  Default workload: B=1, H=32, N=8192, d=128, causal,
bf16 (the headline shape).  ``detail.decode`` adds the split-key-range forward
(fa_fwd_splitkv) on a decode step of 8 x 32 heads, one query against 16384
cached keys, with its HBM roofline, and ``detail.decode_fp8`` the same step
against an FP8 cache (fa_fwd_splitkv_fp8) (skip both with --no-decode), and
``detail.fp8_forward`` the FP8 forward (fa_fwd_fp8) on the headline shape
against the FP8 peak (skip with --no-fp8); ``detail.head_dim_256.fp8_forward``
the FP8 forward on the head dim 256 shape.
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

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense fp8 MFMA (twice the bf16 rate)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "attention fwd+bwd TFLOP/s and % bf16 MFMA peak, 1×MI355X, N=8192 d=128"
COUNTERS = os.path.join(ROOT, "profiles", "counters_c4.json")
# sources each timed kernel is built from (a counter record is valid only for these)
KERNEL_SOURCES = {
    "fwd_bf16_kernel": ["fa_fwd_bf16.hip", "fa_common.h", "fa_dropout.h"],
    "bwd_bf16_kernel": ["fa_bwd_bf16.hip", "fa_bwd_kv_body.h", "fa_common.h", "fa_dropout.h"],
    "bwd_dq_kernel": ["fa_bwd_dq.hip", "fa_common.h", "fa_dropout.h"],
    "bwd_pre_kernel": ["fa_aux.hip", "fa_common.h"],
    "bwd_bf16_ds_kernel": ["fa_bwd_bf16.hip", "fa_bwd_kv_body.h", "fa_common.h", "fa_dropout.h", "fa_launch.h"],
    "bwd_dq_ds_kernel": ["fa_bwd_dq_ds.hip", "fa_common.h", "fa_launch.h"],
}
DQ_METHODS = {0: "handoff", 1: "recompute", 2: "atomic"}


def ds_buffer_bytes(B, H, N, causal):
    """Bytes of the dS hand-off buffer (the dQ kernel reads each once): per
    head, 64-row query block i keeps 2i + 2 (causal) or ceil(N/32) 32-key
    slices of 4 KB (the diagonal's masked entries included)."""
    nqb, nks = -(-N // 64), -(-N // 32)
    per_head = 4096 * (nqb * (nqb + 1) if causal else nqb * nks)
    return B * H * per_head


def backward_kernels(method, unit, T, ds_bytes, kv_ms, dq_ms, suffix=""):
    """Per backward kernel of a dQ method: (name, ms, bound, algorithmic work
    per launch).  MFMA-bound kernels count the products they compute (unit =
    one N x N x d product); the hand-off's dQ kernel is bound by reading dS,
    and counts dS, K read and dQ written once (T elements each of K and dQ)."""
    if method == "handoff":
        return [("bwd_bf16_ds_kernel" + suffix, kv_ms, "mfma", 4 * unit),      # S, dP, dV, dK (+ dS stores)
                ("bwd_dq_ds_kernel" + suffix, dq_ms, "hbm", ds_bytes + 2 * T * 2)]
    if method == "atomic":
        return [("bwd_bf16_kernel" + suffix, kv_ms, "mfma", 5 * unit),         # ... + dQ atomics
                ("dq_convert_kernel" + suffix, dq_ms, "hbm", T * 4 + T * 2)]
    return [("bwd_bf16_kernel" + suffix, kv_ms, "mfma", 4 * unit),             # S, dP, dV, dK
            ("bwd_dq_kernel" + suffix, dq_ms, "mfma", 3 * unit)]               # S, dP, dQ


# Other instantiations whose HBM bytes the counter summary also records, for
# the detail rooflines: key -> ((template name, head dim, split), sources);
# for a kernel templated on flags alone, its template arguments in place of
# the head dim.
# split: True / False for the forwards' split mode (last template argument
# true) or not, None where the kernel has no such argument.  A decode call is
# a split forward plus the merge kernel.
_FWD, _FP8 = ["fa_fwd_bf16.hip", "fa_common.h", "fa_dropout.h"], ["fa_fwd_fp8.hip", "fa_common.h"]
DETAIL_COUNTERS = {
    "fwd_bf16_dropout_kernel": (("fwd_bf16_dropout_kernel", 128, None), _FWD),
    "bwd256_kernel_d256": (("bwd256_kernel", "true, false, true", None),
                           ["fa_bwd_kv256.hip", "fa_bwd_kv256_body.h", "fa_common.h", "fa_dropout.h", "fa_launch.h"]),
    "bwd_dq_ds_kernel_d256": (("bwd_dq_ds_kernel", 256, None), ["fa_bwd_dq_ds.hip", "fa_common.h", "fa_launch.h"]),
    "fwd_fp8_kernel": (("fwd_fp8_kernel", 128, False), _FP8),
    "fwd_bf16_kernel_split": (("fwd_bf16_kernel", 128, True), _FWD),
    "fwd_fp8_kernel_split": (("fwd_fp8_kernel", 128, True), _FP8),
    "fwd_merge_kernel": (("fwd_merge_kernel", 128, None), ["fa_aux.hip", "fa_common.h"]),
}


def _detail_instance(name, key):
    """Whether a traced kernel name is the DETAIL_COUNTERS entry `key`."""
    (short, d, split), _ = DETAIL_COUNTERS[key]
    head = name.split("(")[0].strip()
    if split is not None and head.endswith("true>") != split:
        return False
    return (f"::{short}<{d}," in head or f"::{short}<{d}>" in head or
            (split is None and f"{len(short)}{short}ILi{d}E" in head))


def decode_traffic(split_key):
    """HBM bytes of one decode call: the split forward plus the merge."""
    a, b = traffic_from_counters(split_key), traffic_from_counters("fwd_merge_kernel")
    return None if a is None or b is None else a + b


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_tiled_attention_online_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_counters(kernel):
    """HBM bytes per launch of `kernel`, from the committed rocprofv3 counter
    summary, or None if absent or taken on other sources."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        c = json.load(f).get(kernel)
    srcs = KERNEL_SOURCES.get(kernel) or DETAIL_COUNTERS.get(kernel, (None, None))[1]
    if not c or not srcs or c.get("source_digest") != source_digest(srcs):
        return None
    return c.get("hbm_bytes_per_launch")


def _read_counter_csv(path):
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        per.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return per


def _headline_instance(name, short):
    """Whether a traced kernel name is `short`'s instantiation on the timed
    path (d = 128): the forward's last template argument selects its split
    mode, which is a different launch, and other head dims are other
    instantiations (mangled names carry the head dim as ILi128E)."""
    head = name.split("(")[0].strip()
    if short not in head or not (f"{short}<128," in head or "ILi128E" in head):
        return False
    return not (short == "fwd_bf16_kernel" and head.endswith("true>"))


def summarize_busy(csv_path, last):
    """Clock and matrix-pipe use per kernel from one rocprofv3 run with
    --kernel-trace --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES: per
    dispatch, GRBM_GUI_ACTIVE (summed over the 8 XCDs) / 8 over the duration
    is the shader clock, and SQ_VALU_MFMA_BUSY_CYCLES over that many cycles
    of every SIMD (4 per CU) is the fraction of cycles the matrix pipes are
    busy.  Averages over the last `last` dispatches of each kernel."""
    import collections
    import csv
    rows = collections.defaultdict(dict)
    for r in csv.DictReader(open(csv_path)):
        d = rows[int(r["Dispatch_Id"])]
        d["name"] = r["Kernel_Name"]
        d["dur"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    per = collections.defaultdict(list)
    for _, d in sorted(rows.items()):
        if "GRBM_GUI_ACTIVE" not in d or "SQ_VALU_MFMA_BUSY_CYCLES" not in d or d["dur"] <= 0:
            continue
        cycles = d["GRBM_GUI_ACTIVE"] / 8
        ghz = cycles / d["dur"]
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * 256 * 4) if cycles else 0.0
        per[_short_name(d["name"])].append((d["dur"] / 1000.0, ghz, busy))
    print("| kernel | dispatches | avg us | clock GHz | MFMA busy (of cycles) | busy x GHz |")
    print("|---|---|---|---|---|---|")
    for name, v in sorted(per.items(), key=lambda kv: -sum(x[0] for x in kv[1][-last:])):
        v = v[-last:]
        us, ghz, busy = (sum(x[i] for x in v) / len(v) for i in range(3))
        if us < 100 or busy == 0.0:   # short or MFMA-free launches: the clock estimate is not meaningful
            continue
        print(f"| `{name}` | {len(v)} | {us:.1f} | {ghz:.2f} | {busy:.3f} | {busy * ghz:.2f} |")


STALL_COUNTERS_A = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
                    "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAIT_ANY")
STALL_COUNTERS_B = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_ACTIVE_INST_MISC",
                    "SQ_WAVES", "GRBM_GUI_ACTIVE")


def summarize_stalls(csv_a, csv_b, last):
    """Issue and stall breakdown per kernel from two rocprofv3 --pmc runs of
    this script (STALL_COUNTERS_A, then STALL_COUNTERS_B; one pass may hold at
    most 8 SQ counters).  Per kernel, averages over its last `last`
    dispatches:
      - instructions per wave (SQ_INSTS_* / SQ_WAVES; SQ_INSTS_VALU counts the
        MFMA instructions too, so the VALU column subtracts them);
      - the VALU issue time those instructions need, at 4 cycles per
        instruction of a 64-lane wave, as a fraction of all SIMD cycles
        (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs): a lower bound on the vector
        pipe's share of the kernel;
      - the matrix pipe's busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over the same);
      - SQ_ACTIVE_INST_ANY, SQ_WAIT_INST_ANY and SQ_WAIT_ANY as fractions of
        SQ_WAVE_CYCLES (the wave issuing; waiting for an instruction to issue,
        its operands or a functional unit; waiting on s_waitcnt or a barrier)."""
    import collections
    import csv
    rows = collections.defaultdict(dict)
    for tag, path in (("a", csv_a), ("b", csv_b)):
        for r in csv.DictReader(open(path)):
            d = rows[(tag, int(r["Dispatch_Id"]))]
            d["name"] = _short_name(r["Kernel_Name"])
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for (tag, _), d in sorted(rows.items()):
        for key, val in d.items():
            if key != "name":
                per[d["name"]][key].append(val)
    out = []
    for name, c in per.items():
        if not all(k in c for k in STALL_COUNTERS_A + STALL_COUNTERS_B):
            continue
        m = {k: sum(v[-last:]) / len(v[-last:]) for k, v in c.items()}
        if m["SQ_INSTS_MFMA"] <= 0 or m["SQ_WAVES"] <= 0 or m["SQ_WAVE_CYCLES"] <= 0:
            continue
        simd_cycles = m["GRBM_GUI_ACTIVE"] / 8 * 1024
        waves = m["SQ_WAVES"]
        valu = m["SQ_INSTS_VALU"] - m["SQ_INSTS_MFMA"]
        wc = m["SQ_WAVE_CYCLES"]
        out.append((simd_cycles, f"| `{name}` | {waves:.0f} | {valu / waves:.0f} | {m['SQ_INSTS_MFMA'] / waves:.0f} | "
                                 f"{m['SQ_INSTS_LDS'] / waves:.0f} | {4 * valu / simd_cycles:.2f} | "
                                 f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.2f} | "
                                 f"{m['SQ_ACTIVE_INST_ANY'] / wc:.2f} | {m['SQ_WAIT_INST_ANY'] / wc:.2f} | "
                                 f"{m['SQ_WAIT_ANY'] / wc:.2f} |"))
    print("| kernel | waves | VALU / wave | MFMA / wave | LDS / wave | VALU issue (of SIMD cycles) | "
          "MFMA busy (of SIMD cycles) | issuing | waiting to issue | waiting (waitcnt, barrier) |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for _, line in sorted(out, key=lambda t: -t[0]):
        print(line)


def summarize_counters(fetch_csv, write_csv, copy_mib, out_json):
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, with --copy-probe-mib) into HBM bytes per launch per kernel.

    The probe copy converts copy_mib MiB of bf16 into fp32, so it reads
    copy_mib MiB and writes 2*copy_mib MiB; each counter is scaled by the
    factor that makes the probe's reading exactly that."""
    fetch, write = _read_counter_csv(fetch_csv), _read_counter_csv(write_csv)
    known_read_kib, known_write_kib = copy_mib * 1024.0, 2 * copy_mib * 1024.0

    def mean(d, key):
        v = d.get(key, [])
        return sum(v) / len(v) if v else None

    # the probe is torch's bf16 -> fp32 conversion kernel (the largest such
    # launch in the run); other conversions have other read/write ratios
    copy = [k for k in fetch if "bfloat16tofloat32" in k.replace("_", "").lower() or
            "bfloat16tofloat32" in k.lower()]
    if not copy:
        raise SystemExit("no bf16 -> fp32 copy kernel in the counter run (was --copy-probe-mib given?)")
    ck = max(copy, key=lambda k: max(fetch[k]["FETCH_SIZE"]))
    f_fetch = known_read_kib / max(fetch[ck]["FETCH_SIZE"])
    f_write = known_write_kib / max(write[ck]["WRITE_SIZE"])
    out = {"copy_probe": {"kernel": ck, "mib": copy_mib, "fetch_factor": round(f_fetch, 4),
                          "write_factor": round(f_write, 4)}}
    rows = []
    wanted = [(short, srcs, lambda k, s=short: _headline_instance(k, s)) for short, srcs in KERNEL_SOURCES.items()]
    wanted += [(name, srcs, lambda k, n=name: _detail_instance(k, n)) for name, (_, srcs) in DETAIL_COUNTERS.items()]
    for short, srcs, match in wanted:
        key = next((k for k in fetch if match(k)), None)
        if key is None or key not in write:
            continue
        fk, wkib = mean(fetch[key], "FETCH_SIZE"), mean(write[key], "WRITE_SIZE")
        hbm = (fk * f_fetch + wkib * f_write) * 1024.0
        out[short] = {"fetch_kib_per_launch": round(fk, 1), "write_kib_per_launch": round(wkib, 1),
                      "hbm_bytes_per_launch": int(hbm), "source_digest": source_digest(srcs)}
        rows.append(f"| {short} | {fk:.0f} | {wkib:.0f} | {hbm / 1e6:.1f} |")
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(f"copy probe {ck}: fetch factor {f_fetch:.4f}, write factor {f_write:.4f}")
    print("| kernel | FETCH_SIZE KiB/launch | WRITE_SIZE KiB/launch | HBM MB/launch (scaled) |")
    print("|---|---|---|---|")
    print("\n".join(rows))


def _short_name(name):
    """A traced kernel name without its argument list (torch kernels by their
    function name)."""
    short = name.split("(")[0].replace("void ", "")
    if "at::native" in short:
        short = "torch " + short.split("::")[2].split("<")[0]
    return short[:70]


def summarize_trace(trace_csv, last):
    """Markdown table of kernel durations (us) from a rocprofv3 kernel trace:
    all launches, and the last `last` launches of each kernel, which are the
    timed steps when the traced command is this script with --steps last."""
    import csv
    per = {}
    for r in csv.DictReader(open(trace_csv)):
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), d))
    print(f"| kernel | launches | avg us (all) | avg us (last {last}) | min us | max us |")
    print("|---|---|---|---|---|---|")
    for name, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        ds = [d for _, d in sorted(v)]
        tail = ds[-last:]
        print(f"| `{_short_name(name)}` | {len(ds)} | {sum(ds) / len(ds):.1f} | {sum(tail) / len(tail):.1f} | "
              f"{min(ds):.1f} | {max(ds):.1f} |")


def cpu_baseline(w, x, budget_s=12.0):
    """Time the fp64 oracle on whole heads of the same workload until the
    budget is spent (at least one head); credited-FLOP rate in TFLOP/s.
    Also returns the heads done and the oracle's results for them."""
    from oracle import ref
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    fwd1, bwd1 = w.flops()
    per_head = (fwd1 + bwd1) / (w.B * w.H)
    done, t0 = 0, time.perf_counter()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    results = {}
    while done < len(heads):
        b, h = heads[done]
        results.update(ref.forward_backward(x["q"], x["k"], x["v"], x["do"], w.scale, w.causal,
                                            heads=[(b, h)]))
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    base = {"value": round(per_head * done / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads of the same workload (B=1,H=1,N={w.N},d={w.d}, "
                      f"causal={w.causal}), fp64 materialised fwd+bwd, {dt:.1f} s"}
    return base, heads[:done], results


def cpu_single_core(gen, budget_s=8.0):
    """The oracle on one core (BLAS held to one thread) on whole heads of
    the c1, c2 and c3 workloads: seconds per head and credited TFLOP/s, with
    at most budget_s / 3 seconds per workload (at least one head each)."""
    from threadpoolctl import threadpool_limits
    from oracle import ref
    out = {}
    with threadpool_limits(limits=1):
        for key in ("c1", "c2", "c3"):
            w = gen.workload(key)
            B, H, N, d = w.shape
            x = gen.make_inputs(w, shape=(1, 1, N, d), seed=w.seed)
            fwd1, bwd1 = w.flops()
            per_head = (fwd1 + bwd1) / (B * H)
            done, t0 = 0, time.perf_counter()
            while True:
                ref.forward_backward(x["q"], x["k"], x["v"], x["do"], w.scale, w.causal)
                done += 1
                if time.perf_counter() - t0 > budget_s / 3:
                    break
            dt = time.perf_counter() - t0
            out[w.name] = {"s_per_head": round(dt / done, 4), "heads": done,
                           "tflops": round(per_head * done / dt / 1e12, 6), "cores": 1}
    return out


# the parity bar of the test suite: fp32 max-abs 1e-4; bf16 max-abs 2e-2 * max|ref|
# (max|ref| taken as at least 1e-2); LSE max-abs 1e-3
def oracle_check(w, heads, want, got):
    """Max errors of the timed run's outputs against the oracle on the heads
    the CPU baseline computed, and whether they meet the parity bar."""
    import numpy as np
    errs, ok = {}, True
    for n in ("o", "lse", "dq", "dk", "dv"):
        worst = 0.0
        for (b, h) in heads:
            g = got[n][b, h].float().cpu().numpy().astype(np.float64)
            r = want[(b, h)][n]
            err = float(np.abs(g - r).max())
            if n == "lse":
                tol = 1e-3
            elif w.dtype == "fp32":
                tol = 1e-4
            else:
                tol = 2e-2 * max(1e-2, float(np.abs(r).max()))
            ok = ok and err <= tol
            worst = max(worst, err / tol)
        errs[n] = round(worst, 4)
    return {"heads": len(heads), "first_head": list(heads[0]), "last_head": list(heads[-1]),
            "max_err_over_tolerance": errs, "within_tolerance": ok}


def decode_measurement(fa, gen, torch, dev, stream, with_oracle, reps=50, oracle_budget_s=4.0):
    """The split-key-range forward (fa_fwd_splitkv) on the decode workload:
    time per call from HIP events on the launch stream, its HBM roofline on the
    algorithmic bytes (K, V and Q read once, O and LSE written once), and,
    unless disabled, the oracle on whole heads as a check and a timed CPU
    baseline in the same unit."""
    import numpy as np
    w = gen.DECODE
    x = gen.make_decode_inputs(w.B, w.H, w.Nq, w.Nk, w.d, seed=w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v)
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    nbytes = fa.fa_fwd_splitkv_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, 0)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    sp = stream.cuda_stream

    def call():
        st = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w.B,
                               w.H, w.Nq, w.Nk, w.d, w.causal, w.scale, 0, ws.data_ptr(), ws.numel(), sp,
                               fa.FA_BF16, fa.FA_LAYOUT_BHND)
        if st != 0:
            raise fa.FAError(st, "fa_fwd_splitkv")

    for _ in range(10):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    algo = w.kv_bytes() + 2 * w.B * w.H * w.Nq * w.d * 2 + 4 * w.B * w.H * w.Nq
    gbs = algo / (ms * 1e-3) / 1e9
    res = {"workload": w.name,
           "config": {"B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "causal": w.causal,
                      "scale": w.scale, "num_splits": "auto",
                      "inputs": f"N(0,{w.sigma_qk}^2) q,k; N(0,{w.sigma_v}^2) v; seed {w.seed}"},
           "us_per_call": round(ms * 1e3, 2), "calls": reps,
           "roofline": {"kernel": "fwd_bf16_kernel (split mode) + fwd_merge_kernel", "bound": "hbm",
                        "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": decode_traffic("fwd_bf16_kernel_split"),
                        "algorithmic_bytes": int(algo)}}
    if with_oracle:
        from oracle import ref
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
        done, worst, t0 = 0, {"o": 0.0, "lse": 0.0}, time.perf_counter()
        while done < len(heads):
            b, h = heads[done]
            r = ref.forward_rect(x["q"], x["k"], x["v"], w.scale, w.causal, heads=[(b, h)])[(b, h)]
            worst["o"] = max(worst["o"], float(np.abs(got_o[b, h] - r["o"]).max())
                             / (2e-2 * max(1e-2, float(np.abs(r["o"]).max()))))
            worst["lse"] = max(worst["lse"], float(np.abs(got_l[b, h] - r["lse"]).max()) / 1e-3)
            done += 1
            if time.perf_counter() - t0 > oracle_budget_s:
                break
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(algo * done / len(heads) / dt / 1e9, 3), "unit": "GB/s",
                               "kind": "oracle",
                               "sample": f"{done} of {len(heads)} heads, fp64 materialised forward, {dt:.1f} s"}
        res["oracle_check"] = {"heads": done, "max_err_over_tolerance": {n: round(v, 4) for n, v in worst.items()},
                               "within_tolerance": all(v <= 1.0 for v in worst.values())}
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return res


def decode_fp8_measurement(fa, gen, torch, dev, stream, with_oracle, reps=50, oracle_budget_s=4.0):
    """fa_fwd_splitkv_fp8 on the decode workload with e4m3fn q, k, v (an FP8
    key/value cache): time per call, HBM roofline on the algorithmic bytes
    (K, V, Q read once at one byte per element; O bf16 and LSE written once),
    and the oracle on whole heads within the FP8 bound."""
    import numpy as np
    w = gen.DECODE
    xq = gen.make_fp8_inputs((w.B, w.H, w.Nq, w.d), seed=w.seed, sigma_qk=w.sigma_qk)
    xk = gen.make_fp8_inputs((w.B, w.H, w.Nk, w.d), seed=w.seed + 100, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v)
    q8, k8, v8 = (torch.from_numpy(a).to(dev) for a in (xq["q8"], xk["k8"], xk["v8"]))
    o = torch.empty((w.B, w.H, w.Nq, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    nbytes = fa.fa_fwd_splitkv_fp8_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, 0)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    sp = stream.cuda_stream
    dq, dk, dv = xq["descale_q"], xk["descale_k"], xk["descale_v"]

    def call():
        st = fa.fa_fwd_splitkv_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   w.B, w.H, w.Nq, w.Nk, w.d, w.causal, w.scale, dq, dk, dv, 0, ws.data_ptr(),
                                   ws.numel(), sp, fa.FA_LAYOUT_BHND)
        if st != 0:
            raise fa.FAError(st, "fa_fwd_splitkv_fp8")

    for _ in range(10):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    algo = w.kv_bytes() // 2 + w.B * w.H * w.Nq * w.d * (1 + 2) + 4 * w.B * w.H * w.Nq
    gbs = algo / (ms * 1e-3) / 1e9
    res = {"workload": w.name.replace("bf16", "fp8"), "dtype": "fp8 e4m3fn q, k, v; bf16 out",
           "us_per_call": round(ms * 1e3, 2), "calls": reps,
           "roofline": {"kernel": "fwd_fp8_kernel (split mode) + fwd_merge_kernel", "bound": "hbm",
                        "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": decode_traffic("fwd_fp8_kernel_split"),
                        "algorithmic_bytes": int(algo)}}
    if with_oracle:
        from oracle import ref
        got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        worst, done, t0 = {"o": 0.0, "lse": 0.0}, 0, time.perf_counter()
        for b, h in heads:
            r = ref.forward_rect(xq["q"], xk["k"], xk["v"], w.scale, w.causal, heads=[(b, h)])[(b, h)]
            vmax = float(np.abs(xk["v"][b, h]).max())
            tol = (2.0 ** -4 + w.Nk * 2.0 ** -17) * vmax + 2.0 ** -9 * float(np.abs(r["o"]).max())
            worst["o"] = max(worst["o"], float(np.abs(got_o[b, h] - r["o"]).max()) / tol)
            worst["lse"] = max(worst["lse"], float(np.abs(got_l[b, h] - r["lse"]).max()) / 1e-3)
            done += 1
            if time.perf_counter() - t0 > oracle_budget_s:
                break
        res["oracle_check"] = {"heads": done, "max_err_over_tolerance": {n: round(v, 4) for n, v in worst.items()},
                               "within_tolerance": all(v <= 1.0 for v in worst.values())}
    del q8, k8, v8, o, lse, ws
    torch.cuda.empty_cache()
    return res


def fp8_measurement(fa, gen, torch, dev, stream, w, with_oracle, reps=30, oracle_budget_s=4.0,
                    counters="fwd_fp8_kernel"):
    """The FP8 forward (fa_fwd_fp8) on workload w's shape with e4m3fn inputs:
    time per call from HIP events on the launch stream, credited forward
    FLOPs (4*B*H*N^2*d, halved for causal) against the dense FP8 peak, and,
    unless disabled, the oracle on whole heads (the values the codes stand
    for) within the bound the tests use.  `counters` names the stored
    rocprofv3 counter entry for this shape (None: none taken)."""
    import numpy as np
    B, H, N, d = w.shape
    x = gen.make_fp8_inputs((B, H, N, d), seed=w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_vdo)
    q8, k8, v8 = (torch.from_numpy(x[n]).to(dev) for n in ("q8", "k8", "v8"))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    sp = stream.cuda_stream

    def call():
        st = fa.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                           w.causal, w.scale, x["descale_q"], x["descale_k"], x["descale_v"], sp,
                           fa.FA_LAYOUT_BHND)
        if st != 0:
            raise fa.FAError(st, "fa_fwd_fp8")

    for _ in range(10):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    fl = w.flops()[0]
    tf = fl / (ms * 1e-3) / 1e12
    res = {"workload": w.name.replace("bf16", "fp8"), "dtype": "fp8 e4m3fn in, bf16 out",
           "descales": [x["descale_q"], x["descale_k"], x["descale_v"]],
           "us_per_call": round(ms * 1e3, 2), "calls": reps, "tflops": round(tf, 3),
           "roofline": {"kernel": "fwd_fp8_kernel", "bound": "mfma", "achieved": round(tf, 3),
                        "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                        "traffic": traffic_from_counters(counters) if counters else None}}
    if with_oracle:
        from oracle import ref
        got_o, got_l = o.float().cpu().numpy(), lse.cpu().numpy()
        worst, done, t0 = {"o": 0.0, "lse": 0.0}, 0, time.perf_counter()
        for h in range(H):
            r = ref.forward_rect(x["q"], x["k"], x["v"], w.scale, w.causal, heads=[(0, h)])[(0, h)]
            vmax = float(np.abs(x["v"][0, h]).max())
            tol = (2.0 ** -4 + N * 2.0 ** -17) * vmax + 2.0 ** -9 * float(np.abs(r["o"]).max())
            worst["o"] = max(worst["o"], float(np.abs(got_o[0, h] - r["o"]).max()) / tol)
            worst["lse"] = max(worst["lse"], float(np.abs(got_l[0, h] - r["lse"]).max()) / 1e-3)
            done += 1
            if time.perf_counter() - t0 > oracle_budget_s:
                break
        res["oracle_check"] = {"heads": done, "max_err_over_tolerance": {n: round(v, 4) for n, v in worst.items()},
                               "within_tolerance": all(v <= 1.0 for v in worst.values())}
    del q8, k8, v8, o, lse
    torch.cuda.empty_cache()
    return res


def head_dim_256_measurement(fa, torch, stream, with_oracle, reps=10):
    """Head dim 256 at the headline's credited FLOPs: causal 1 x 16 x 8192 x
    256, bf16 (inputs from a seeded device generator).  Per-stage times from
    HIP events on the launch stream, credited TFLOP/s, the dominant kernel
    against the dense bf16 peak (its algorithmic FLOPs: 4 products of
    2*B*H*N^2*d/2 for dK/dV, 3 for the recomputing dQ kernel, 2 for the
    forward; the hand-off's dQ kernel is HBM-bound and reported in GB/s) and,
    unless disabled, 256 query rows of head (0, 0) (O, LSE) against the
    oracle."""
    import numpy as np
    B, H, N, d = 1, 16, 8192, 256
    scale = 1.0 / 16.0
    g = torch.Generator(device=stream.device).manual_seed(256)
    q, k, v, do = (torch.randn((B, H, N, d), generator=g, device=stream.device).to(torch.bfloat16) for _ in range(4))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = fa.workspace(q)
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()
    lay = fa.FA_LAYOUT_BHND

    def step(ev=None):
        calls = [
            lambda: fa.fa_fwd(P(q), P(k), P(v), P(o), P(lse), B, H, N, d, True, scale, sp, fa.FA_BF16, lay),
            lambda: fa.fa_bwd_preprocess(P(o), P(do), P(lse), B, H, N, d, scale, P(ws), ws.numel(), sp, fa.FA_BF16,
                                         lay),
            lambda: fa.fa_bwd_dkdv(P(q), P(k), P(v), P(do), P(lse), P(dk), P(dv), B, H, N, d, True, scale, P(ws),
                                   ws.numel(), sp, fa.FA_BF16, lay),
            lambda: fa.fa_bwd_dq(P(q), P(k), P(v), P(do), P(lse), P(dq), B, H, N, d, True, scale, P(ws), ws.numel(),
                                 sp, fa.FA_BF16, lay),
        ]
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i].record(stream)
            st = c()
            if st != 0:
                raise fa.FAError(st, "head dim 256 step")
        if ev is not None:
            ev[4].record(stream)

    for _ in range(3):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    avg = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in evs) / reps
    fwd_ms, pre_ms, kv_ms, dq_ms = avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4)
    unit = 2 * B * H * N * N * d / 2    # one causal N x N x d product
    fwd_fl, bwd_fl = 2 * unit, 5 * unit
    method = DQ_METHODS[fa.fa_bwd_dq_method(B, H, N, d, True, fa.FA_BF16, ws.numel(), 0)]
    bk = backward_kernels(method, unit, B * H * N * d, ds_buffer_bytes(B, H, N, True), kv_ms, dq_ms)
    # d = 256 has its own dK/dV kernel (bwd256_kernel<causal, dropout, dS stores>)
    bk = [("bwd256_kernel" if n.startswith("bwd_bf16") else n, t, bound, w) for n, t, bound, w in bk]
    kernels = {"fwd_bf16_kernel": (fwd_ms, 2 * unit)}
    kernels.update({n: (t, fl) for n, t, bound, fl in bk if bound == "mfma"})
    hbm = {n: (t, b) for n, t, bound, b in bk if bound == "hbm"}
    dom = max(kernels, key=lambda n: kernels[n][0])
    tf = kernels[dom][1] / (kernels[dom][0] * 1e-3) / 1e12
    bwd_ms = pre_ms + kv_ms + dq_ms
    res = {"workload": "bf16_b1h16_n8192_d256_causal", "dq_mode": method, "fwd_ms": round(fwd_ms, 4),
           "bwd_ms": round(bwd_ms, 4), "bwd_dkdv_ms": round(kv_ms, 4), "bwd_dq_ms": round(dq_ms, 4),
           "bwd_frac_peak": round(bwd_fl / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "tflops": round((fwd_fl + bwd_fl) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 3),
           "kernel_tflops": {n: round(f / (t * 1e-3) / 1e12, 3) for n, (t, f) in kernels.items()},
           "hbm_kernels": {n: {"achieved_gbs": round(b / (t * 1e-3) / 1e9, 1),
                               "frac": round(b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                               "traffic": traffic_from_counters(n + "_d256") if n + "_d256" in DETAIL_COUNTERS
                               else None} for n, (t, b) in hbm.items()},
           "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(tf, 3), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic_from_counters(dom + "_d256") if dom + "_d256" in DETAIL_COUNTERS
                        else None}}
    if with_oracle:
        from oracle import ref
        rows = 256
        q0, k0, v0 = (t[0, 0].float().cpu().numpy().astype(np.float64) for t in (q, k, v))
        p, _, want_l = ref.softmax_rows(ref.scores(q0[:rows], k0, scale, True))
        want_o = p @ v0
        e_o = float(np.abs(o[0, 0, :rows].float().cpu().numpy() - want_o).max()) / (
            2e-2 * max(1e-2, float(np.abs(want_o).max())))
        e_l = float(np.abs(lse[0, 0, :rows].cpu().numpy() - want_l).max()) / 1e-3
        res["oracle_check"] = {"rows": f"head (0,0), query rows 0..{rows - 1}",
                               "max_err_over_tolerance": {"o": round(e_o, 4), "lse": round(e_l, 4)},
                               "within_tolerance": e_o <= 1.0 and e_l <= 1.0}
    del q, k, v, do, o, dq, dk, dv, lse, ws
    torch.cuda.empty_cache()
    return res


DROP_T = 26   # drop probability 26/256 (about 0.1) for the dropout measurement


def dropout_measurement(fa, torch, stream, w, q, k, v, do, ws, plain_fwd_ms, plain_bwd_ms, with_oracle, x=None,
                        reps=20):
    """Attention with dropout (fa_fwd_dropout, fa_bwd_dropout) on the
    headline tensors: per-call times from HIP events on the launch stream,
    credited FLOPs as for the plain step (dropout adds no products), the
    forward kernel against the dense bf16 peak, the cost over the plain path,
    and, unless disabled, the first 1024 query rows of head (0, 0) against the
    dropout oracle (O, LSE)."""
    import numpy as np
    B, H, N, d = w.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    sp = stream.cuda_stream
    seed, offset = 0x5EED0123456789AB, 3
    P = lambda t: t.data_ptr()

    def fwd():
        st = fa.fa_fwd_dropout(P(q), P(k), P(v), P(o), P(lse), B, H, N, d, w.causal, w.scale, DROP_T, seed, offset,
                               sp, fa.FA_LAYOUT_BHND)
        if st != 0:
            raise fa.FAError(st, "fa_fwd_dropout")

    def bwd():
        st = fa.fa_bwd_dropout(P(q), P(k), P(v), P(o), P(do), P(lse), P(dq), P(dk), P(dv), B, H, N, d, w.causal,
                               w.scale, DROP_T, seed, offset, P(ws), ws.numel(), sp, fa.FA_LAYOUT_BHND)
        if st != 0:
            raise fa.FAError(st, "fa_bwd_dropout")

    for _ in range(5):
        fwd()
        bwd()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
    torch.cuda.synchronize()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    fwd_fl, bwd_fl = w.flops()
    fwd_tf = fwd_fl / (fwd_ms * 1e-3) / 1e12
    res = {"workload": w.name + "_dropout", "drop_t": DROP_T, "drop_probability": DROP_T / 256,
           "generator": "Philox4x32-10, one call per 4x4 block", "fwd_ms": round(fwd_ms, 4),
           "bwd_ms": round(bwd_ms, 4), "step_ms": round(fwd_ms + bwd_ms, 4), "reps": reps,
           "tflops": round((fwd_fl + bwd_fl) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 3),
           "fwd_over_plain": round(fwd_ms / plain_fwd_ms, 3), "bwd_over_plain": round(bwd_ms / plain_bwd_ms, 3),
           "roofline": {"kernel": "fwd_bf16_dropout_kernel", "bound": "mfma", "achieved": round(fwd_tf, 3),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic_from_counters("fwd_bf16_dropout_kernel")}}
    if with_oracle and x is not None:
        from oracle import dropout as drop
        from oracle import ref
        rows = min(N, 1024)
        q0, k0, v0 = (np.asarray(x[n][0, 0], dtype=np.float64) for n in ("q", "k", "v"))
        keep = drop.keep_mask(0, seed, offset, DROP_T, N, N, row0=0, rows=rows)
        s = ref.scores(q0[:rows], k0, w.scale, w.causal, row0=0)
        p, _, want_l = ref.softmax_rows(s)
        want_o = drop.keep_scale(DROP_T) * np.where(keep, p, 0.0) @ v0
        got_o = o[0, 0, :rows].float().cpu().numpy()
        got_l = lse[0, 0, :rows].cpu().numpy()
        e_o = float(np.abs(got_o - want_o).max()) / (2e-2 * max(1e-2, float(np.abs(want_o).max())))
        e_l = float(np.abs(got_l - want_l).max()) / 1e-3
        res["oracle_check"] = {"rows": f"head (0,0), query rows 0..{rows - 1}",
                               "max_err_over_tolerance": {"o": round(e_o, 4), "lse": round(e_l, 4)},
                               "within_tolerance": e_o <= 1.0 and e_l <= 1.0}
    del o, lse, dq, dk, dv
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c4", help="c1..c5 (default c4, the headline shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 forwards on the headline and head dim 256 shapes (reported under detail)")
    ap.add_argument("--no-d256", action="store_true",
                    help="skip the head dim 256 step (1 x 16 x 8192 x 256, reported under detail)")
    ap.add_argument("--no-dropout", action="store_true",
                    help="skip the dropout forward and backward on the headline shape (reported under detail)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the split-key-range forward on the decode workload (reported under detail)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="write a scratch buffer of this many MiB between timed steps (untimed), so "
                         "that the 256 MB last-level cache holds no inputs; the step time is then the "
                         "sum of the per-step event intervals instead of the bracketing wall clock")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(the calibration kernel for rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_MIB"),
                    help="write profiles/counters_c4.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-busy", nargs=2, metavar=("PMC_CSV", "LAST"),
                    help="print per-kernel clock and MFMA-busy fraction from a rocprofv3 --kernel-trace --pmc "
                         "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES run and exit")
    ap.add_argument("--summarize-stalls", nargs=3, metavar=("PMC_A_CSV", "PMC_B_CSV", "LAST"),
                    help="print per-kernel instruction counts, pipe use and stall fractions from two "
                         "rocprofv3 --pmc runs (the counters of STALL_COUNTERS_A, then STALL_COUNTERS_B) and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "LAST"),
                    help="print per-kernel durations from a rocprofv3 --kernel-trace CSV: over all "
                         "launches and over the last LAST launches (the timed steps) and exit")
    args = ap.parse_args()
    if args.summarize_busy:
        summarize_busy(args.summarize_busy[0], int(args.summarize_busy[1]))
        return 0
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], int(args.summarize_trace[1]))
        return 0
    if args.summarize_stalls:
        summarize_stalls(args.summarize_stalls[0], args.summarize_stalls[1], int(args.summarize_stalls[2]))
        return 0
    if args.summarize_counters:
        fcsv, wcsv, mib = args.summarize_counters
        summarize_counters(fcsv, wcsv, float(mib), COUNTERS)
        return 0
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported (the (batch, head) "
              "pairs are independent, so several GPUs would each take a share of them)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import exact_tiled_attention_online_amd as fa
    from exact_tiled_attention_online_amd import inputs as gen

    w = gen.workload(args.workload)
    dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP32
    x = gen.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v, do = (torch.from_numpy(x[n]).to(dev).to(dtype) for n in ("q", "k", "v", "do"))
    B, H, N, d = w.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = fa.workspace(q)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    P = lambda t: t.data_ptr()
    lay = fa.FA_LAYOUT_BHND

    def check(st, what):
        if st != 0:
            raise fa.FAError(st, what)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        check(fa.fa_fwd(P(q), P(k), P(v), P(o), P(lse), B, H, N, d, w.causal, w.scale, sp, code, lay), "fa_fwd")
        if ev is not None:
            ev[1].record(stream)
        check(fa.fa_bwd_preprocess(P(o), P(do), P(lse), B, H, N, d, w.scale, P(ws), ws.numel(), sp, code,
                                   lay), "fa_bwd_preprocess")
        if ev is not None:
            ev[2].record(stream)
        check(fa.fa_bwd_dkdv(P(q), P(k), P(v), P(do), P(lse), P(dk), P(dv), B, H, N, d, w.causal,
                             w.scale, P(ws), ws.numel(), sp, code, lay), "fa_bwd_dkdv")
        if ev is not None:
            ev[3].record(stream)
        check(fa.fa_bwd_dq(P(q), P(k), P(v), P(do), P(lse), P(dq), B, H, N, d, w.causal, w.scale,
                           P(ws), ws.numel(), sp, code, lay), "fa_bwd_dq")
        if ev is not None:
            ev[4].record(stream)

    scratch = torch.empty(args.flush_mib * (1 << 20), dtype=torch.uint8, device=dev) if args.flush_mib else None
    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if scratch is not None:
            scratch.fill_(i & 0xFF)
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = sorted(e[0].elapsed_time(e[4]) for e in events)
    if scratch is None:
        ms_step = (t1 - t0) * 1e3 / args.steps
    else:
        ms_step = sum(step_ms) / len(step_ms)

    # calibration: a vendor-library bf16 GEMM of 8192^3 on the same device
    # (hipBLASLt through torch), the practical dense-MFMA rate of this part
    # under its power limit, reported beside the nominal peak
    gemm_tflops = None
    if dtype == torch.bfloat16:
        ga = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        gb = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        for _ in range(5):
            gc = ga @ gb
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(20):
            gc = ga @ gb
        g1.record(stream)
        torch.cuda.synchronize()
        gemm_tflops = 2 * 8192 ** 3 / (g0.elapsed_time(g1) / 20 * 1e-3) / 1e12
        del ga, gb, gc

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty(n, dtype=torch.float32, device=dev)
        dst.copy_(src)          # reads copy_probe_mib MiB, writes twice that
        torch.cuda.synchronize()
        del src, dst

    def avg(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in events) / len(events)

    fwd_ms, pre_ms, kv_ms, dq_ms = avg(0, 1), avg(1, 2), avg(2, 3), avg(3, 4)
    fwd_fl, bwd_fl = w.flops()
    unit = bwd_fl / 5.0             # one N x N x d product: 2*B*H*N^2*d FLOPs (halved if causal)
    value = (fwd_fl + bwd_fl) / (ms_step * 1e-3) / 1e12
    bwd_ms = pre_ms + kv_ms + dq_ms
    method = DQ_METHODS[fa.fa_bwd_dq_method(B, H, N, d, w.causal, code, ws.numel(), 0)]
    elem = 2 if w.dtype == "bf16" else 4
    T = B * H * N * d
    # algorithmic work per launch of each kernel: the products it computes
    # (MFMA-bound) or the bytes it must move (HBM-bound)
    bk = backward_kernels(method, unit, T, ds_buffer_bytes(B, H, N, w.causal), kv_ms, dq_ms)
    mfma_k = {"fwd_bf16_kernel": (fwd_ms, 2 * unit)}                  # S, P V
    mfma_k.update({n: (t, fl) for n, t, bound, fl in bk if bound == "mfma"})
    hbm_k = {n: (t, b) for n, t, bound, b in bk if bound == "hbm"}
    dom = max(mfma_k, key=lambda k: mfma_k[k][0])
    dom_ms, dom_fl = mfma_k[dom]
    achieved = dom_fl / (dom_ms * 1e-3) / 1e12
    pre_bytes = 2 * T * elem + 12 * B * H * N
    headline = args.workload == "c4" and w.dtype == "bf16"
    traffic = traffic_from_counters(dom) if headline else None
    pre_traffic = traffic_from_counters("bwd_pre_kernel") if headline else None
    props = torch.cuda.get_device_properties(0)
    bwd_frac = bwd_fl / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS

    out = {
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
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "scale": w.scale, "inputs": f"N(0,{w.sigma_qk}^2) q,k; N(0,{w.sigma_vdo}^2) v,dO; seed {w.seed}"},
        "roofline": {"kernel": dom, "bound": "mfma",
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
        "target": {"what": "backward credited TFLOP/s (10*B*H*N^2*d, halved causal, over bwd_ms) / dense bf16 peak",
                   "value": round(bwd_frac, 4), "bar": 0.40, "met": bool(bwd_frac >= 0.40),
                   "bwd_ms": round(bwd_ms, 4), "bwd_ms_at_bar": round(bwd_fl / (0.40 * PEAK_BF16_TFLOPS * 1e12) * 1e3, 4)},
        "detail": {
            "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
            "bwd_preprocess_ms": round(pre_ms, 4), "bwd_dkdv_ms": round(kv_ms, 4),
            "bwd_dq_ms": round(dq_ms, 4), "dq_mode": method,
            "fwd_tflops": round(fwd_fl / (fwd_ms * 1e-3) / 1e12, 3),
            "bwd_tflops": round(bwd_fl / (bwd_ms * 1e-3) / 1e12, 3),
            "fwd_frac_peak": round(fwd_fl / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "bwd_frac_peak": round(bwd_fl / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernel_tflops": {k: round(f / (t * 1e-3) / 1e12, 3) for k, (t, f) in mfma_k.items()},
            "hbm_kernels": {k: {"bound": "hbm", "achieved": round(b / (t * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(b / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                "algorithmic_bytes": int(b),
                                "traffic": traffic_from_counters(k) if headline else None}
                            for k, (t, b) in hbm_k.items()},
            "preprocess_roofline": {"kernel": "bwd_pre_kernel", "bound": "hbm",
                                    "achieved": round(pre_bytes / (pre_ms * 1e-3) / 1e9, 1),
                                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(pre_bytes / (pre_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                    "traffic": pre_traffic},
            "step_ms_median": round(step_ms[len(step_ms) // 2], 4),
            "step_ms_min": round(step_ms[0], 4),
            "flush_mib": args.flush_mib,
            "gpu": torch.cuda.get_device_name(0),
            "compute_units": props.multi_processor_count,
            "vendor_gemm_bf16_tflops": round(gemm_tflops, 1) if gemm_tflops else None,
            "dominant_kernel_frac_of_vendor_gemm": round(achieved / gemm_tflops, 4) if gemm_tflops else None,
            "peak_from_cus_at_2p4ghz": round(props.multi_processor_count * 4096 * 2.4e9 / 1e12, 1),
        },
    }
    if not args.no_dropout and dtype == torch.bfloat16:
        out["detail"]["dropout"] = dropout_measurement(fa, torch, stream, w, q, k, v, do, ws, fwd_ms, bwd_ms,
                                                       not args.no_cpu_baseline, x)
    if not args.no_d256 and dtype == torch.bfloat16:
        out["detail"]["head_dim_256"] = head_dim_256_measurement(fa, torch, stream, not args.no_cpu_baseline)
        if not args.no_fp8:
            w256 = gen.Workload("bf16_b1h16_n8192_d256_causal", 1, 16, 8192, 256, "bf16", True, 1.0, 1.0, 256)
            out["detail"]["head_dim_256"]["fp8_forward"] = fp8_measurement(
                fa, gen, torch, dev, stream, w256, not args.no_cpu_baseline, counters=None)
    if not args.no_fp8 and B == 1 and d == 128:
        out["detail"]["fp8_forward"] = fp8_measurement(fa, gen, torch, dev, stream, w, not args.no_cpu_baseline)
    if not args.no_decode:
        out["detail"]["decode"] = decode_measurement(fa, gen, torch, dev, stream, not args.no_cpu_baseline)
        out["detail"]["decode_fp8"] = decode_fp8_measurement(fa, gen, torch, dev, stream, not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        base, heads, ref = cpu_baseline(w, x)
        out["cpu_baseline"] = base
        out["detail"]["cpu_single_core"] = cpu_single_core(gen)
        out["detail"]["oracle_check"] = oracle_check(w, heads, ref, {"o": o, "lse": lse, "dq": dq,
                                                                    "dk": dk, "dv": dv})
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
