"""Summaries of rocprofv3 output for the profiles/ folder.

  stats    kernel statistics of a --kernel-trace --stats run (top kernels by
           total time)
  traffic  HBM bytes per launch of one kernel from two --pmc runs (FETCH_SIZE,
           then WRITE_SIZE), each calibrated by what the same counter reads
           for the plain 1 GiB device copy that `bench.py --pmc-copy` runs
           (the copy reads 1 GiB and writes 1 GiB per launch)
  mfma     MFMA-busy fraction per kernel from one --pmc run of
           SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and
           SQ_INSTS_VALU_MFMA_MOPS_BF16: busy SIMD cycles over active GPU
           cycles x SIMD_NUM, and the MFMA FLOPs those instructions did
  lds      per kernel from one --pmc run of SQ_LDS_IDX_ACTIVE,
           SQ_LDS_BANK_CONFLICT, SQ_VALU_MFMA_BUSY_CYCLES, TA_BUSY_avr and
           GRBM_GUI_ACTIVE: LDS busy cycles over active cycles x CU count,
           the share of those cycles stalled on bank conflicts, the texture
           address unit's busy fraction and the MFMA-busy fraction

Usage:
  python -m layer_streamed_amd.prof_summary stats STATS_CSV OUT_MD --title T --command C
  python -m layer_streamed_amd.prof_summary traffic FETCH_CSV WRITE_CSV OUT_MD \\
      --kernel NAME --flops-per-launch F --command-fetch C1 --command-write C2
  python -m layer_streamed_amd.prof_summary mfma PMC_CSV OUT_MD --title T --command C
  python -m layer_streamed_amd.prof_summary lds PMC_CSV OUT_MD --title T --command C [--note N]
"""
import argparse
import csv
import hashlib
import os
import re
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 1 << 30


def short(name):
    name = re.sub(r"^void ", "", name)
    name = name.replace("mt::(anonymous namespace)::", "")
    return re.sub(r"\(.*$", "", name)


def gemm_sources_sha256():
    src = os.path.join(ROOT, "layer_streamed_amd", "csrc")
    return hashlib.sha256(open(os.path.join(src, "gemm.hip"), "rb").read()
                          + open(os.path.join(src, "common.h"), "rb").read()).hexdigest()


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"# {args.title}", "", "Command (from the repository root):", "",
           f"    {args.command}", "", f"Top kernels by total time ({total / 1e6:.1f} ms of "
           "kernel time in the run):", "",
           "| kernel | calls | avg (us) | total (ms) | % |", "|---|---|---|---|---|"]
    for r in rows[: args.top]:
        out.append(f"| {short(r['Name'])[:72]} | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['TotalDurationNs']) / 1e6:.1f} | "
                   f"{100 * float(r['TotalDurationNs']) / total:.2f} |")
    open(args.out, "w").write("\n".join(out) + "\n")


def _per_dispatch(path, counter):
    """(short kernel name, dispatch id) -> counter value summed over dimensions."""
    agg = defaultdict(float)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        agg[(short(r["Kernel_Name"]), int(r["Dispatch_Id"]))] += float(r["Counter_Value"])
    return agg


def traffic(args):
    fetch = _per_dispatch(args.fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(args.write_csv, "WRITE_SIZE")

    def pick(agg, pred):
        return [v for (n, _), v in sorted(agg.items(), key=lambda kv: kv[0][1]) if pred(n)]

    is_copy = lambda n: "copyBuffer" in n  # noqa: E731
    is_k = lambda n: n == args.kernel  # noqa: E731
    kf, kw = pick(fetch, is_k), pick(write, is_k)
    # the calibration copies are the 1 GiB ones: far larger than any other
    # device copy of the run (weight initialisation makes many small ones)
    cf, cw = pick(fetch, is_copy), pick(write, is_copy)
    cf = [v for v in cf if v > 0.5 * max(cf)]
    cw = [v for v in cw if v > 0.5 * max(cw)]
    assert kf and kw, f"no dispatch of {args.kernel} in the counter files"
    assert cf and cw, "no calibration copy (bench.py --pmc-copy) in the counter files"
    # counters are in KiB; the copy moves COPY_BYTES each way
    f_scale = COPY_BYTES / (sum(cf) / len(cf) * 1024)
    w_scale = COPY_BYTES / (sum(cw) / len(cw) * 1024)
    fb = sum(kf) / len(kf) * 1024 * f_scale
    wb = sum(kw) / len(kw) * 1024 * w_scale
    out = [f"# HBM traffic of {args.kernel} ({args.workload})", "",
           f"kernel: {args.kernel}", "",
           "Commands (two passes, one counter each, from the repository root):", "",
           f"    {args.command_fetch}", f"    {args.command_write}", "",
           f"Dispatches of the kernel: {len(kf)} (FETCH_SIZE pass), {len(kw)} (WRITE_SIZE pass); "
           f"calibration copies: {len(cf)} / {len(cw)}.", "",
           "| | FETCH_SIZE (KiB, mean) | WRITE_SIZE (KiB, mean) |", "|---|---|---|",
           f"| kernel | {sum(kf) / len(kf):.1f} | {sum(kw) / len(kw):.1f} |",
           f"| copy 1 GiB | {sum(cf) / len(cf):.1f} | {sum(cw) / len(cw):.1f} |", "",
           f"Calibration (the copy reads and writes 1 GiB per launch): FETCH_SIZE scale "
           f"{f_scale:.4f}, WRITE_SIZE scale {w_scale:.4f} (bytes = KiB x 1024 x scale).", "",
           "Per launch (mean over the kernel's dispatches):",
           f"- fetched from HBM: {fb / 1e9:.3f} GB",
           f"- written to HBM: {wb / 1e9:.3f} GB",
           f"- traffic_bytes_per_launch: {int(fb + wb)}"]
    if args.flops_per_launch:
        out.append(f"- algorithmic FLOPs per launch: {args.flops_per_launch:.4g} "
                   f"(arithmetic intensity {args.flops_per_launch / (fb + wb):.0f} FLOP/byte "
                   f"of measured traffic)")
    if args.note:
        out += ["", args.note]
    out += ["", f"source_sha256: {gemm_sources_sha256()}",
            "(sha256 of gemm.hip followed by common.h when the counters were taken; the "
            "benchmark reports this traffic only while the sources still hash to it and the "
            "kernel is still the dominant one.)"]
    open(args.out, "w").write("\n".join(out) + "\n")


def _gpu_agent(csv_path):
    """(XCD count, SIMD count) of the GPU agent from the run's agent-info file."""
    info = os.path.join(os.path.dirname(csv_path),
                        os.path.basename(csv_path).replace("counter_collection", "agent_info"))
    for r in csv.DictReader(open(info)):
        if r["Agent_Type"] == "GPU":
            return int(r["Num_Xcc"]), int(r["Simd_Count"])
    raise SystemExit(f"no GPU agent in {info}")


def mfma(args):
    busy, active, mops, dur = (defaultdict(float) for _ in range(4))
    names = {}
    for r in csv.DictReader(open(args.csv)):
        key = int(r["Dispatch_Id"])
        names[key] = short(r["Kernel_Name"])
        dur[key] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])  # ns
        v = float(r["Counter_Value"])
        c = r["Counter_Name"]
        if c == "SQ_VALU_MFMA_BUSY_CYCLES":
            busy[key] += v
        elif c == "GRBM_GUI_ACTIVE":
            active[key] += v
        elif c == "SQ_INSTS_VALU_MFMA_MOPS_BF16":
            mops[key] += v
    xcc, simds = _gpu_agent(args.csv)
    # the file holds one value per dispatch, GRBM_GUI_ACTIVE summed over the
    # XCDs: per XCD (the clock that every SIMD shares) it is that / xcc
    by = defaultdict(lambda: [0, 0.0, 0.0, 0.0, 0.0])
    for key, n in names.items():
        g = by[n]
        g[0] += 1
        g[1] += busy[key]
        g[2] += active[key] / xcc
        g[3] += mops[key] * 512
        g[4] += dur[key]
    tot_busy = sum(g[1] for g in by.values())
    tot_active = sum(g[2] for g in by.values())
    rows = sorted(by.items(), key=lambda kv: -kv[1][2])
    out = [f"# {args.title}", "", "Command (from the repository root):", "", f"    {args.command}", "",
           "MFMA-busy fraction = SQ_VALU_MFMA_BUSY_CYCLES (summed over SIMDs) / (active cycles "
           f"x {simds} SIMDs), per kernel over its dispatches, where active cycles = "
           f"GRBM_GUI_ACTIVE / {xcc} (the file sums it over the {xcc} XCDs); clock = active "
           "cycles / kernel duration; MFMA FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. Kernels "
           "on other streams may overlap a dispatch.", "",
           f"All kernels of the run: MFMA busy {100 * tot_busy / max(tot_active * simds, 1):.1f}% "
           f"of {tot_active:.4g} active cycles.", "",
           "| kernel | dispatches | active cycles | clock (GHz) | MFMA busy | MFMA TFLOP (counted) | "
           "TFLOP/s (counted / time) |",
           "|---|---|---|---|---|---|---|"]
    for n, (k, b, a, f, t) in rows[: args.top]:
        out.append(f"| {n[:72]} | {k} | {a:.4g} | {a / max(t, 1):.2f} | "
                   f"{100 * b / max(a * simds, 1):.1f}% | {f / 1e12:.2f} | "
                   f"{f / max(t, 1) / 1e3:.0f} |")
    open(args.out, "w").write("\n".join(out) + "\n")


def lds(args):
    keys = ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_BUSY_CYCLES", "TA_BUSY_avr",
            "GRBM_GUI_ACTIVE")
    val = defaultdict(lambda: defaultdict(float))
    names = {}
    for r in csv.DictReader(open(args.csv)):
        key = int(r["Dispatch_Id"])
        names[key] = short(r["Kernel_Name"])
        if r["Counter_Name"] in keys:
            val[key][r["Counter_Name"]] += float(r["Counter_Value"])
    xcc, simds = _gpu_agent(args.csv)
    cus = simds // 4
    by = defaultdict(lambda: defaultdict(float))
    for key, n in names.items():
        g = by[n]
        g["n"] += 1
        for k in keys:
            g[k] += val[key][k]
    rows = sorted(by.items(), key=lambda kv: -kv[1]["GRBM_GUI_ACTIVE"])
    out = [f"# {args.title}", "", "Command (from the repository root):", "", f"    {args.command}", "",
           f"Per kernel over its dispatches, with active cycles = GRBM_GUI_ACTIVE / {xcc} (the file "
           f"sums it over the {xcc} XCDs): LDS busy = SQ_LDS_IDX_ACTIVE / (active cycles x {cus} "
           "CUs) (indexed LDS operations, i.e. the reads; the direct global-to-LDS copies are not "
           "counted); bank-conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; TA busy = "
           "TA_BUSY_avr (the mean over the texture address units) / active cycles; MFMA busy = "
           f"SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x {simds} SIMDs).", ""]
    if args.note:
        out += [args.note, ""]
    out += ["| kernel | dispatches | LDS busy | bank-conflict share | TA busy | MFMA busy |",
            "|---|---|---|---|---|---|"]
    for n, g in rows[: args.top]:
        act = g["GRBM_GUI_ACTIVE"] / xcc
        out.append(f"| {n[:72]} | {int(g['n'])} | {100 * g['SQ_LDS_IDX_ACTIVE'] / max(act * cus, 1):.1f}% | "
                   f"{100 * g['SQ_LDS_BANK_CONFLICT'] / max(g['SQ_LDS_IDX_ACTIVE'], 1):.1f}% | "
                   f"{100 * g['TA_BUSY_avr'] / max(act, 1):.1f}% | "
                   f"{100 * g['SQ_VALU_MFMA_BUSY_CYCLES'] / max(act * simds, 1):.1f}% |")
    open(args.out, "w").write("\n".join(out) + "\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("out")
    a.add_argument("--title", required=True)
    a.add_argument("--command", required=True)
    a.add_argument("--top", type=int, default=24)
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("out")
    b.add_argument("--kernel", required=True)
    b.add_argument("--workload", default="Qwen2.5-7B shape, B 16 x T 1024")
    b.add_argument("--flops-per-launch", type=float, default=0.0)
    b.add_argument("--command-fetch", required=True)
    b.add_argument("--command-write", required=True)
    b.add_argument("--note", default="")
    c = sub.add_parser("mfma")
    c.add_argument("csv")
    c.add_argument("out")
    c.add_argument("--title", required=True)
    c.add_argument("--command", required=True)
    c.add_argument("--top", type=int, default=20)
    d = sub.add_parser("lds")
    d.add_argument("csv")
    d.add_argument("out")
    d.add_argument("--title", required=True)
    d.add_argument("--command", required=True)
    d.add_argument("--note", default="")
    d.add_argument("--top", type=int, default=20)
    args = ap.parse_args()
    {"stats": stats, "traffic": traffic, "mfma": mfma, "lds": lds}[args.cmd](args)


if __name__ == "__main__":
    main()
