"""Throughput of the scaled low-precision GEMM path on one MI355X.

One step = one pass of the path over one batch of synthetic input: quantize
the bf16 activations on the GPU (row-wise E4M3, per-tensor E4M3 or NVFP4,
per the workload), then one gemm_scaled launch with its fused epilogue.
Weights are quantized once, before timing (they are pre-quantized in
inference, as in AstrAI's E4M3 benchmark on pre-quantized NT operands).  Three input/weight
buffer sets rotate from step to step so the working set exceeds the 256 MB
last-level cache.

Prints ONE JSON line: whole-step TFLOP/s (value), the GEMM kernel's roofline
position (its launch durations measured with events on the launch stream
inside the timed region), and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synthetic import WORKLOADS  # noqa: E402

METRIC = "TFLOP/s and % of dense FP8 MFMA peak, scaled GEMM at T=4096 (and T=1024)"
DEFAULT_WORKLOAD = "fp8_row_swiglu_t4096"

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
PEAK_TFLOPS = {"fp8": 5000.0, "f16": 2500.0}
HBM_GBS = 8000.0

# the kernels of one gemm_scaled call (the GEMM, its split-K reduction) and
# the planner that picks their launches (split, tail, grid), which changes
# the traffic as much as the kernels do; by the plan's kernel (0, 2: FP8
# tiles, 1: NVFP4 tiles, 3: decode width)
KERNEL_NAMES = {0: "gemm_fp8_kernel", 1: "gemm_nvfp4_kernel", 2: "gemm_fp8_half_kernel", 3: "gemm_narrow_kernel"}
GEMM_SOURCES = {
    "gemm_fp8_kernel": ["spg_gemm_fp8.hip", "spg_gemm_common.h", "spg_common.h", "spg_splitk.hip", "spg_api.hip"],
    "gemm_fp8_half_kernel": ["spg_gemm_fp8.hip", "spg_gemm_common.h", "spg_common.h", "spg_api.hip"],
    "gemm_nvfp4_kernel": ["spg_gemm_nvfp4.hip", "spg_gemm_common.h", "spg_common.h", "spg_splitk.hip",
                          "spg_api.hip"],
    "gemm_narrow_kernel": ["spg_gemm_narrow.hip", "spg_gemm_common.h", "spg_common.h", "spg_api.hip"],
}


def kernel_of(wl) -> str:
    """Name of the main GEMM kernel the planner picks for a workload (the
    library's planner, called on the host; MI355X's 256 compute units)."""
    import scaled_precision_gemm_amd as spg
    p = spg.gemm_plan(wl.M, wl.N, wl.K, wl.fmt, wl.epilogue, batch=wl.batch, units=256)
    return KERNEL_NAMES[p["kernel"]]


def code_only(text: str) -> str:
    """Source text without comments and blank space differences: what the
    compiler sees (a comment edit does not change the kernel)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(kname: str, read=None) -> str:
    """Hash of the sources of a GEMM kernel's calls, comments ignored.  `read`
    maps a csrc file name to its text (default: the working tree)."""
    h = hashlib.sha256()
    for f in GEMM_SOURCES[kname]:
        if read is None:
            with open(os.path.join(ROOT, "scaled_precision_gemm_amd", "csrc", f)) as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(code_only(text).encode())
    return h.hexdigest()[:16]


def gemm_bytes(wl) -> int:
    """Algorithmic HBM bytes of one GEMM launch: read A and W codes (and the
    NVFP4 scale planes), read the residual, write the bf16 output once."""
    b = wl.batch
    if wl.fmt == "nvfp4":
        ab = wl.M * wl.K // 2 + wl.M * wl.K // 16
        wb = wl.N * wl.K // 2 + wl.N * wl.K // 16
    else:
        ab = wl.M * wl.K
        wb = wl.N * wl.K
    out = 2 * wl.M * wl.n_out
    res = 2 * (1 if wl.bias else wl.M) * wl.n_out if wl.epilogue == "add" else 0
    return b * (ab + wb + out + res)


def quantize_bytes(wl) -> int:
    """Algorithmic bytes of the step's activation quantization: bf16 in, codes
    and scales out (read once: per-tensor FP8 and NVFP4 read the activations
    twice, a partial-maximum pass and then the encode pass, but the minimum
    is one read)."""
    elems = wl.batch * wl.M * wl.K
    if wl.fmt == "e4m3_row":
        return 3 * elems + 4 * wl.batch * wl.M
    if wl.fmt == "e4m3_tensor":
        return 3 * elems + 4 * wl.batch
    return 2 * elems + elems // 2 + elems // 16 + 4


def operator_bytes(M, N, K, n_out, residual: bool, fmt: str) -> int:
    """Bytes of the quantize + GEMM operator as ninfer PR #160's operator
    table counts them: bf16 activations in, weight codes and scales, bf16
    output, bf16 residual."""
    if fmt == "nvfp4":
        w = N * K // 2 + N * K // 16
    else:
        w = N * K + 4 * N
    return 2 * M * K + w + 2 * M * n_out + (2 * M * n_out if residual else 0)


def traffic_from_profiles(wl, name):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    only when it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(name)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("kernel_source_hash") != kernel_source_hash(kernel_of(wl)):
        return None
    return rec.get("hbm_bytes_per_launch")


def _read_csv(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def summarize_profiles(name, stats_dir, fetch_dir, write_dir, command="", counters_dir=None, ea_dir=None,
                       l2_dir=None):
    """Write profiles/<kernel>_<workload>.md (rocprofv3 kernel statistics, HBM
    traffic per launch and, given a counters run, MFMA and LDS utilisation)
    and the traffic record bench.py reports.

    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the GEMM are scaled by what
    the same counters read for the plain copy dispatch of known size that
    --copy-probe-mib runs in the same process.  MfmaUtil and LdsUtil are
    rocprofv3's derived metrics (MFMA busy cycles over SIMD cycles, LDS busy
    cycles over CU cycles, at the clock the kernel actually ran).

    ea_dir (a run of TCC_EA0_RDREQ_sum and its 32-, 64- and 128-byte parts
    with the same copy probe) checks FETCH_SIZE against raw request counts:
    bytes = 32 n32 + 64 n64 + 128 n128.  l2_dir (TCC_HIT_sum, TCC_MISS_sum,
    TCC_EA0_RDREQ_DRAM_sum, TCC_BUBBLE_sum) gives the L2 hit rate and the
    share of the read requests addressed to memory (DRAM) rather than to
    another die or IO."""
    wl = WORKLOADS[name]
    kname = kernel_of(wl)
    stats = _read_csv(_find(stats_dir, "kernel_stats.csv"))
    lines = ["| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        short = r["Name"].replace("void ", "").replace("spg::(anonymous namespace)::", "").split("(")[0]
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")

    # One gemm_scaled call is one to three dispatches (main tiles, a K-split
    # tail, its reduction); bench.py's events bracket the whole call.  The
    # timed steps are the last `--steps` calls of the traced run.
    lines_ = command.strip().splitlines()

    def run_counts(line):
        """(timed steps, all gemm_scaled calls) of the bench run on command
        line `line` (the bench's defaults where a flag is not given)."""
        toks = lines_[line].split() if len(lines_) > line else []
        val = {"--steps": 200, "--warmup": 10, "--settle-launches": 150}
        for i, a in enumerate(toks[:-1]):
            if a in val:
                val[a] = int(toks[i + 1])
        return val["--steps"], val["--steps"] + val["--warmup"] + val["--settle-launches"]

    steps, n_calls = run_counts(0)
    timed_avg_us = None
    try:
        trace = _read_csv(_find(stats_dir, "kernel_trace.csv"))
        durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in
                sorted(trace, key=lambda r: int(r["Start_Timestamp"]))
                if "gemm_" in r["Kernel_Name"] or "splitk_reduce" in r["Kernel_Name"]]
        per_call = len(durs) // n_calls
        if per_call >= 1 and len(durs) == per_call * n_calls:
            timed_avg_us = float(np.sum(durs[-steps * per_call:])) / steps / 1e3
    except FileNotFoundError:
        pass

    def per_call(d, counter, line):
        """Counter value of each gemm_scaled call (summed over its dispatches)
        and of the copy dispatches, from the run of command line `line`."""
        _, calls = run_counts(line)
        rows = sorted(_read_csv(_find(d, "counter_collection.csv")), key=lambda r: int(r["Dispatch_Id"]))
        vals = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter
                and ("gemm_" in r["Kernel_Name"] or "splitk_reduce" in r["Kernel_Name"])]
        k = max(1, len(vals) // calls)
        gemm = [sum(vals[i:i + k]) for i in range(0, k * calls, k)] if len(vals) == k * calls else vals
        copy = [(float(r["Counter_Value"]), int(r["Grid_Size"])) for r in rows
                if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower()]
        return gemm, copy

    g_fetch, c_fetch = per_call(fetch_dir, "FETCH_SIZE", 1)
    g_write, c_write = per_call(write_dir, "WRITE_SIZE", 2)
    copy_bytes = None
    for i, a in enumerate(command.split()):
        if a == "--copy-probe-mib":
            copy_bytes = int(command.split()[i + 1]) << 20
    f_read = (max(v for v, _ in c_fetch) * 1024 / copy_bytes) if (c_fetch and copy_bytes) else 1.0
    f_write = (max(v for v, _ in c_write) * 1024 / copy_bytes) if (c_write and copy_bytes) else 1.0
    rd = float(np.median(g_fetch)) * 1024 / f_read
    wr = float(np.median(g_write)) * 1024 / f_write
    util = None
    if counters_dir:
        # duration-weighted over the dispatches of each call, median over the
        # timed calls (command line 4 names its --steps / --warmup)
        st, n_all = run_counts(3)
        rows = sorted(_read_csv(_find(counters_dir, "counter_collection.csv")), key=lambda r: int(r["Dispatch_Id"]))
        util = {}
        for metric in ("MfmaUtil", "LdsUtil"):
            disp = [(float(r["Counter_Value"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in rows
                    if r["Counter_Name"] == metric and ("gemm_" in r["Kernel_Name"] or "splitk_reduce" in r["Kernel_Name"])]
            k = max(1, len(disp) // n_all)
            calls = [disp[i:i + k] for i in range(0, len(disp) - k + 1, k)][-st:]
            call_vals = [sum(v * d for v, d in c) / max(1, sum(d for _, d in c)) for c in calls]
            util[metric] = float(np.median(call_vals)) if call_vals else None
        util["dispatches_per_call"] = k

    ea = None
    if ea_dir:
        ea = {}
        for ctr in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum"):
            g, c = per_call(ea_dir, ctr, 4)
            ea[ctr] = (float(np.median(g)), max(v for v, _ in c) if c else None)

        def req_bytes(i):
            n = [ea[f"TCC_EA0_RDREQ_{b}B_sum"][i] for b in (32, 64, 128)]
            return None if any(v is None for v in n) else 32.0 * n[0] + 64.0 * n[1] + 128.0 * n[2]
        ea["gemm_read_bytes"] = req_bytes(0)
        ea["copy_read_bytes"] = req_bytes(1)
        ea["copy_bytes"] = copy_bytes
        ea["req_128_share"] = ea["TCC_EA0_RDREQ_128B_sum"][0] / max(1.0, ea["TCC_EA0_RDREQ_sum"][0])
    l2 = None
    if l2_dir:
        l2 = {}
        for ctr in ("TCC_HIT_sum", "TCC_MISS_sum", "TCC_EA0_RDREQ_DRAM_sum", "TCC_BUBBLE_sum"):
            g, _ = per_call(l2_dir, ctr, 5)
            l2[ctr] = float(np.median(g))
        l2["hit_rate"] = l2["TCC_HIT_sum"] / max(1.0, l2["TCC_HIT_sum"] + l2["TCC_MISS_sum"])
        if ea:
            l2["dram_share"] = l2["TCC_EA0_RDREQ_DRAM_sum"] / max(1.0, ea["TCC_EA0_RDREQ_sum"][0])

    rec = {
        "kernel": kname, "workload": name, "kernel_source_hash": kernel_source_hash(kname),
        "hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
        "hbm_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": gemm_bytes(wl),
        "fetch_scale": f_read, "write_scale": f_write, "rocprof_avg_call_us": timed_avg_us,
    }
    if util:
        rec["mfma_util_pct"] = util["MfmaUtil"]
        rec["lds_util_pct"] = util["LdsUtil"]
    if ea:
        rec["ea_read_bytes_per_launch"] = ea["gemm_read_bytes"]
        rec["copy_probe_ea_read_bytes"] = ea["copy_read_bytes"]
    if l2:
        rec["l2_hit_rate"] = l2["hit_rate"]
        if "dram_share" in l2:
            rec["ea_read_request_dram_share"] = l2["dram_share"]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    allrec = json.load(open(tpath)) if os.path.exists(tpath) else {}
    allrec[name] = rec
    with open(tpath, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
    md = os.path.join(ROOT, "profiles", f"{kname}_{name}.md")
    with open(md, "w") as fh:
        fh.write(f"# {kname} on {name} (M={wl.M}, N={wl.N}, K={wl.K}, batch={wl.batch}, {wl.fmt}, {wl.epilogue})\n\n")
        fh.write(f"Kernel statistics, `rocprofv3 --kernel-trace --stats` (one MI355X):\n\n")
        fh.write("\n".join(lines) + "\n\n")
        if timed_avg_us is not None:
            fh.write(f"GPU time of one gemm_scaled call (all its dispatches: main tiles, K-split tail and "
                     f"reduction where the plan has them) averaged over the {steps} timed steps alone, the "
                     f"last {steps} calls of the kernel trace (the warmup calls above include the power "
                     f"controller's throttling dip): {timed_avg_us:.1f} us\n\n")
        fh.write(f"HBM traffic of one gemm_scaled call, all its dispatches (`rocprofv3 --pmc FETCH_SIZE`, "
                 f"then `--pmc WRITE_SIZE`, median over calls), scaled by the counters' reading for a plain copy of "
                 f"{(copy_bytes or 0) >> 20} MiB (read scale {f_read:.4f}, write scale {f_write:.4f}):\n\n")
        fh.write(f"- read  {rd / 1e6:.1f} MB, write {wr / 1e6:.1f} MB, total {(rd + wr) / 1e6:.1f} MB\n")
        fh.write(f"- algorithmic (A and W codes once, residual once, output once): {gemm_bytes(wl) / 1e6:.1f} MB\n")
        fh.write(f"- kernel source hash {rec['kernel_source_hash']}\n\n")
        if timed_avg_us:
            fh.write(f"Achieved over the call: {wl.flops / (timed_avg_us * 1e-6) / 1e12:.0f} TFLOP/s; HBM "
                     f"{(rd + wr) / (timed_avg_us * 1e-6) / 1e9:.0f} GB/s measured, "
                     f"{gemm_bytes(wl) / (timed_avg_us * 1e-6) / 1e9:.0f} GB/s algorithmic (of 8000).\n\n")
        if ea:
            cb = ea["copy_bytes"] or 0
            fh.write(f"Read side from raw L2-to-memory (EA) request counts by size (`--pmc TCC_EA0_RDREQ_sum "
                     f"TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum`, same copy probe): "
                     f"the {cb / 1e6:.1f} MB copy issues requests for {(ea['copy_read_bytes'] or 0) / 1e6:.1f} MB, "
                     f"which FETCH_SIZE counts {1 / f_read if f_read else 0:.2f}x (hence its read scale); the GEMM "
                     f"call's requests come to {ea['gemm_read_bytes'] / 1e6:.1f} MB "
                     f"({ea['gemm_read_bytes'] / gemm_bytes(wl):.2f}x the algorithmic bytes; the scaled FETCH_SIZE "
                     f"gives {rd / 1e6:.1f} MB), {100 * ea['req_128_share']:.0f}% of them 128-byte requests.  "
                     f"These counters sit at the L2: whether the memory side serves a request from its "
                     f"last-level cache or from HBM is not visible to them.\n\n")
        if l2:
            fh.write(f"L2 (`--pmc TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_DRAM_sum TCC_BUBBLE_sum`): hit rate "
                     f"{100 * l2['hit_rate']:.1f}%"
                     + (f"; {100 * l2['dram_share']:.1f}% of the read requests addressed to memory (DRAM) rather "
                        f"than another die or IO" if "dram_share" in l2 else "") + ".\n\n")
        if util:
            fh.write(f"Utilisation (`rocprofv3 --pmc MfmaUtil LdsUtil`, duration-weighted over the call's "
                     f"{util['dispatches_per_call']} dispatch(es), median over the timed calls): MFMA busy "
                     f"{util['MfmaUtil']:.1f}% of SIMD cycles, LDS busy {util['LdsUtil']:.1f}% of CU cycles, "
                     f"both at the clock the kernels ran at.\n\n")
        fh.write("Commands (run from the repository root on the GPU box with `TMPDIR=/tmp` exported; each "
                 "under `timeout`):\n\n")
        fh.write("```\n" + command.strip() + "\n```\n")
    print(f"wrote {md} and {tpath}")


def run_probes(torch, spg):
    """The device's own ceilings, measured after the timed steps: MFMA-only
    rates (E4M3 32x32x64 and f16 32x32x16 on register operands) with the
    shader clock they ran at, and a read-only HBM stream over 1 GiB."""
    units = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    out = {}
    for kind, name, iters in ((0, "fp8", 40000), (1, "f16", 80000)):
        spg.probe_mfma(kind, iters // 10, 2 * units)            # settle
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            _, clocks, flops = spg.probe_mfma(kind, iters, 2 * units)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            c = clocks.cpu().tolist()
            sclk = (c[1] - c[0]) / max(1, c[3] - c[2]) * 0.1
            if best is None or ms < best[0]:
                best = (ms, flops, sclk)
        out[f"mfma_{name}_tflops"] = round(best[1] / (best[0] * 1e-3) / 1e12, 1)
        out[f"mfma_{name}_sclk_ghz"] = round(best[2], 3)
    buf = torch.empty((1 << 30,), dtype=torch.uint8, device="cuda")
    spg.probe_read(buf, 8 * units)
    best = None
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        spg.probe_read(buf, 8 * units)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    out["hbm_read_gbs"] = round(buf.numel() / (best * 1e-3) / 1e9, 1)
    del buf
    out["note"] = ("after the timed steps, same device: MFMA-only loops on random register operands "
                   "(4 independent chains per wave, 2 workgroups of 4 waves per CU), best of 3; "
                   "sclk from s_memtime against the 100 MHz s_memrealtime; 1 GiB read-only stream")
    return out


def to_dev(x16, torch):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).view(torch.bfloat16).cuda()


def cpu_baseline(wl, A16, W16, R16, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same step:
    quantize `rows` activation rows and compute their whole output rows
    (weights quantized beforehand, outside the timed part, as on the GPU)."""
    import oracle
    if wl.batch > 1:
        A16, W16 = A16[0], W16[0]
    if wl.fmt == "e4m3_row":
        Wq, sw = oracle.quantize_rowwise(W16)
    elif wl.fmt == "e4m3_tensor":
        Wq, sw = oracle.quantize_tensor(W16)
        sw = sw[0]
        sa_t = oracle.amax(A16) / np.float32(448.0)
    else:
        tw = oracle.nvfp4_tensor_scale(W16)
        Wq, Ws = oracle.quantize_block16_rows(W16, tw)
        ta = oracle.nvfp4_tensor_scale(A16)

    def step(rows):
        a = np.ascontiguousarray(A16[:rows])
        if R16 is None:
            r = None
        elif wl.bias:
            r = np.broadcast_to(R16, (rows, wl.n_out))
        else:
            r = np.ascontiguousarray(R16[:rows])
        if wl.fmt == "e4m3_row":
            qa, sa = oracle.quantize_rowwise(a)
            D, Da = oracle.gemm_e4m3_sums(qa, Wq)
            oracle.epilogue(wl.epilogue, D, Da, sa, sw, r)
        elif wl.fmt == "e4m3_tensor":
            qa = oracle.quantize_rows_with_scale(a, sa_t)
            D, Da = oracle.gemm_e4m3_sums(qa, Wq)
            oracle.epilogue(wl.epilogue, D, Da, sa_t, sw, r)
        else:
            qa, sa = oracle.quantize_block16_rows(a, ta)
            D, Da = oracle.gemm_nvfp4_sums(qa, sa, Wq, Ws)
            oracle.epilogue(wl.epilogue, D, Da, ta, tw, r)

    # the oracle parallelizes over rows: calibrate on one row per thread,
    # then time a whole number of such rounds filling the budget
    per = oracle.threads()
    t0 = time.perf_counter()
    step(per)
    one = max(time.perf_counter() - t0, 1e-4)
    rows = int(min(wl.M, per * max(1, round(budget_s / one))))
    t0 = time.perf_counter()
    step(rows)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * wl.N * wl.K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"{rows} of {wl.M} token rows of one product: quantize + all {wl.n_out} outputs "
                  f"({wl.epilogue}), fp64, {dt:.1f} s",
        "seconds": dt,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    # MI355X's power controller throttles hard a few launches after an idle
    # spell and needs ~100 launches (~60 ms) of this load to settle.  The
    # settle phase runs before the warmup, is reported as its own field
    # (settle_launches, settle_ms) and is never counted as warmup.
    ap.add_argument("--settle-launches", type=int, default=150,
                    help="steps run (and reported) before the warmup so the power controller settles")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not have the timed GEMM launches record their shader clock")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--sets", type=int, default=3, help="rotating input/weight buffer sets")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true", help="skip the MFMA-only and HBM read probes")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before timing, run one plain bf16->f16 copy of this many MiB (the reference "
                         "dispatch for calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="no GPU work: turn rocprofv3 output of this workload (STATS_DIR FETCH_DIR WRITE_DIR "
                         "[COUNTERS_DIR [EA_DIR L2_DIR]]) into profiles/ summaries")
    ap.add_argument("--command", default="", help="with --summarize: the command line that produced the runs")
    args = ap.parse_args()

    if args.summarize:
        if len(args.summarize) not in (3, 4, 6):
            ap.error("--summarize takes STATS_DIR FETCH_DIR WRITE_DIR [COUNTERS_DIR [EA_DIR L2_DIR]]")
        d = args.summarize
        summarize_profiles(args.workload, d[0], d[1], d[2], command=args.command,
                           counters_dir=d[3] if len(d) >= 4 else None, ea_dir=d[4] if len(d) == 6 else None,
                           l2_dir=d[5] if len(d) == 6 else None)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU sharding or collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    import scaled_precision_gemm_amd as spg

    wl = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    A16, W16, R16 = wl.inputs()
    sets = max(1, args.sets)

    # ---- device buffers: `sets` rotated activation / weight sets ------------
    A0, W0 = to_dev(A16, torch), to_dev(W16, torch)
    R = to_dev(R16, torch) if R16 is not None else None
    acts, weights = [], []
    for s in range(sets):
        shift = 977 * s
        A = A0 if s == 0 else torch.roll(A0, shifts=shift, dims=-2).contiguous()
        W = W0 if s == 0 else torch.roll(W0, shifts=shift, dims=-2).contiguous()
        if wl.fmt == "e4m3_row":
            wq = spg.quantize_rowwise(W)
        elif wl.fmt == "e4m3_tensor":
            wq = spg.quantize_tensor(W)
        else:
            wq = spg.quantize_block16(W, layout="blocked")
        acts.append(A)
        weights.append(wq)
        del W
    del A0, W0
    torch.cuda.synchronize()

    # activation-side buffers, reused every step
    if wl.fmt == "e4m3_row":
        qa = torch.empty(wl.a_shape(), dtype=torch.uint8, device="cuda")
        sa = torch.empty((wl.M,), dtype=torch.float32, device="cuda")
    out = torch.empty((wl.batch, wl.M, wl.n_out) if wl.batch > 1 else (wl.M, wl.n_out),
                      dtype=torch.bfloat16, device="cuda")
    # a split-N output (fused input projections): one tensor per column segment
    segs = [torch.empty((wl.M, w), dtype=torch.bfloat16, device="cuda") for w in wl.split] if wl.split else None
    ws = None

    def step(i, cp=None):
        nonlocal ws
        A = acts[i % sets]
        w = weights[i % sets]
        if wl.fmt == "e4m3_row":
            spg.quantize_rowwise(A, out=qa, scale=sa)
            ev[i][1].record()
            spg.gemm_scaled(qa, sa, w[0], w[1], wl.epilogue, residual=R, out=None if segs else out,
                            workspace=ws, clock_probe=cp, out_split=segs)
        elif wl.fmt == "e4m3_tensor":
            q, s = spg.quantize_tensor(A)
            ev[i][1].record()
            spg.gemm_scaled(q, s, w[0], w[1], wl.epilogue, fmt="e4m3_tensor", out=out, workspace=ws,
                            clock_probe=cp)
        else:
            q, bs, t = spg.quantize_block16(A, layout="blocked")
            ev[i][1].record()
            spg.gemm_scaled(q, bs, w[0], w[1], wl.epilogue, residual=R, fmt="nvfp4", out=out,
                            tscale_a=t, tscale_w=w[2], workspace=ws, clock_probe=cp, scale_layout="blocked")

    # workspace sized once by the library's own query, reused every step
    plan = spg.gemm_plan(wl.M, wl.N, wl.K, wl.fmt, wl.epilogue, batch=wl.batch)
    a_codes = qa if wl.fmt == "e4m3_row" else None
    if a_codes is None:
        a_codes = torch.empty(wl.a_shape() if wl.fmt != "nvfp4" else (wl.M, wl.K // 2), dtype=torch.uint8,
                              device="cuda")
    ws = spg.gemm_workspace(a_codes, weights[0][0], wl.fmt, wl.epilogue, out=out, residual=R)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty(n // 2, dtype=torch.float16, device="cuda")
        dst.copy_(src)                        # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()
    n_ev = max(args.warmup, args.steps, args.settle_launches, 1)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]

    settle_ms = 0.0
    if args.settle_launches > 0:
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for i in range(args.settle_launches):
            ev[i][0].record()
            step(i)
            ev[i][2].record()
        s1.record(stream)
        torch.cuda.synchronize()
        settle_ms = s0.elapsed_time(s1)
    for i in range(args.warmup):
        ev[i][0].record()
        step(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    # shader clock of each timed step's main GEMM launch, recorded by the
    # kernel itself (first workgroup, at its start and end: two stores)
    clk = None if args.no_clock else torch.zeros((max(args.steps, 1), 4), dtype=torch.int64, device="cuda")

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        ev[i][0].record()
        step(i, clk[i] if clk is not None else None)
        ev[i][2].record()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    gemm_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)]
    quant_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]

    ms_per_step = total_ms / args.steps
    flops = wl.flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_avg = float(np.mean(gemm_ms))
    achieved = flops / (gemm_avg * 1e-3) / 1e12
    peak_key = "f16" if wl.fmt == "nvfp4" else "fp8"
    peak = PEAK_TFLOPS[peak_key]
    # the GEMM is bound by whichever roof its arithmetic intensity reaches
    # first: MFMA above the ridge (peak flops / HBM bandwidth), HBM below
    alg_bytes = gemm_bytes(wl)
    hbm_bound = flops / alg_bytes < peak * 1e12 / (HBM_GBS * 1e9)
    if hbm_bound:
        achieved_v, peak_v, unit = alg_bytes / (gemm_avg * 1e-3) / 1e9, HBM_GBS, "GB/s"
    else:
        achieved_v, peak_v, unit = achieved, peak, "TFLOP/s"
    roofline = {
        "bound": "hbm" if hbm_bound else "mfma",
        "kernel": KERNEL_NAMES[plan["kernel"]],
        "achieved": round(achieved_v, 1),
        "peak": peak_v,
        "unit": unit,
        "frac": round(achieved_v / peak_v, 4),
        "gemm_tflops": round(achieved, 1),
        "traffic": traffic_from_profiles(wl, args.workload),
        "algorithmic_bytes": alg_bytes,
        "flops_per_launch": flops,
        "launch_ms_avg": round(gemm_avg, 4),
        "launch_ms_median": round(float(np.median(gemm_ms)), 4),
        "launch_ms_p10_p90": [round(float(np.percentile(gemm_ms, 10)), 4),
                              round(float(np.percentile(gemm_ms, 90)), 4)],
        "frac_at_median": round((flops / (float(np.median(gemm_ms)) * 1e-3) / 1e12 / peak) if not hbm_bound else
                                (alg_bytes / (float(np.median(gemm_ms)) * 1e-3) / 1e9 / HBM_GBS), 4),
    }
    if clk is not None:
        c = clk.cpu().numpy().astype(np.float64)
        ghz = (c[:, 1] - c[:, 0]) / np.maximum(1.0, c[:, 3] - c[:, 2]) / 10.0
        roofline["sclk_ghz_timed"] = {"median": round(float(np.median(ghz)), 3),
                                      "min": round(float(ghz.min()), 3), "max": round(float(ghz.max()), 3),
                                      "how": "recorded by the main GEMM launch of every timed step (first "
                                             "workgroup: shader-clock against 100 MHz counter, start to end)"}
        roofline["wg0_kernel_cycles_median"] = int(np.median(c[:, 1] - c[:, 0]))
        # the MFMA peak scaled to the clock the timed steps actually ran at
        if not hbm_bound:
            roofline["frac_of_peak_at_timed_sclk"] = round(achieved / (peak * float(np.median(ghz)) / 2.4), 4)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_launches": args.settle_launches,
        "settle_ms": round(settle_ms, 2),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if wl.fmt == "nvfp4" else "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "format": wl.fmt, "epilogue": "add (bf16 bias row)" if wl.bias else wl.epilogue,
            "M": wl.M, "N": wl.N, "K": wl.K, "batch": wl.batch,
            **({"out_split": list(wl.split)} if wl.split else {}),
            "step": "activation quantize + gemm_scaled (weights pre-quantized)",
            "buffer_sets": sets, "plan": plan,
        },
        "pct_fp8_peak": round(100.0 * value / PEAK_TFLOPS["fp8"], 2),
        "quantize_ms_avg": round(float(np.mean(quant_ms)), 4),
        "wall_s_timed": round(wall, 3),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    line["quantize_gbs"] = round(quantize_bytes(wl) / (line["quantize_ms_avg"] * 1e-3) / 1e9, 1)
    if not args.no_probes:
        line["probes"] = run_probes(torch, spg)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(wl, A16, W16, R16, args.cpu_budget)
        line["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in cb.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
