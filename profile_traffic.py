"""rocprofv3 helpers behind the roofline figures that bench.py reports.

    python3 profile_traffic.py launch [--launches N] [--workload W]
        A workload (headline_bf16, the benchmark's, or k256_bf16) launched N
        times back to back, then the calibration copy: torch.bitwise_not over
        a 256 MiB int32 buffer into another (reads 256 MiB, writes 256 MiB).
        Run it once under `rocprofv3 --pmc FETCH_SIZE` and once under
        `rocprofv3 --pmc WRITE_SIZE`.

    python3 profile_traffic.py traffic FETCH_DIR WRITE_DIR --command CMD [--workload W]
        Reads the two counter CSVs, scales the kernel's FETCH_SIZE and
        WRITE_SIZE (KiB per dispatch) by what the same counters read for the
        calibration copy, and writes profiles/traffic_W.json (read by
        bench.py) and a text summary beside it.

    python3 profile_traffic.py counters PMC_DIR --command CMD [--workload W]
        Writes profiles/counters_W.md (and .json) from a `rocprofv3 --pmc`
        run of `launch` with the SQ counters listed in COUNTERS: MFMA busy
        cycles, LDS bank conflicts against LDS instruction cycles, waves and
        the GPU's busy clocks, averaged over the kernel's dispatches.

    python3 profile_traffic.py issue PMC_DIR_A PMC_DIR_B --command CMD [--workload W]
        Writes profiles/counters_issue_W.md (and .json) from two `rocprofv3
        --pmc` runs of `launch` with the two counter lists of ISSUE_COUNTERS:
        the fractions of the waves' cycles spent executing VALU and LDS
        instructions, waiting to issue and waiting for anything, and the
        instruction counts per wave.

    python3 profile_traffic.py stats STATS_DIR --command CMD [--name NAME] [--by-grid]
        Writes profiles/kernel_stats_NAME.md (default headline_bf16) from a
        `rocprofv3 --kernel-trace --stats` run of bench.py; with --by-grid,
        from the per-dispatch trace, one line per kernel and grid size (the
        same kernel launched on two workloads).
"""
import argparse
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

CAL_BYTES = 256 << 20
CAL_KERNEL = "bitwise_not"
PROFILES = os.path.join(ROOT, "profiles")


KERNELS = {"headline_bf16": bench.KERNEL_NAME, "k256_bf16": bench.K256_KERNEL_NAME,
           "fwd_bwd_bf16": "bwd_grads", "fwd_bwd_dk64_bf16": "bwd_grads"}
# The backward's kernels, in launch order: the forward walk that saves each
# chunk's entering state and Delta rows, the reverse walk of the state
# gradient, and the per-chunk gradient kernel.
BWD_KERNELS = ["gdn_fwd_bf16<false, 3, {dk}>", "gdn_fwd_bf16<false, 4, {dk}>", "bwd_grads"]


def launch(n, workload):
    import numpy as np
    import torch
    import gated_deltanet_chunked_chunk_amd as gdn
    import gdn_inputs as gi
    gdn.load()
    dev = torch.device("cuda:0")
    if workload.startswith("fwd_bwd"):
        d = gi.make_config(workload)
        do, dht = gi.make_upstream(d, gi.CONFIGS[workload]["seed"])
        up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        q, k, v, dO = up(d["q"]), up(d["k"]), up(d["v"]), up(do)
        g, b = torch.from_numpy(d["g"]).to(dev), torch.from_numpy(d["beta"]).to(dev)
        dh = torch.from_numpy(dht).to(dev)
        for i in range(n):
            gdn.gdn_chunk_bwd(q, k, v, g, b, dO, dht=dh)
            torch.cuda.synchronize()
            print(f"[launch] backward {i + 1}/{n}", flush=True)
        _calibration_copy(torch, dev)
        return
    if workload == "headline_bf16":
        d = gi.make_config(workload)
        up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
        g, b = torch.from_numpy(d["g"]).to(dev), torch.from_numpy(d["beta"]).to(dev)
    else:
        c = gi.CONFIGS[workload]
        d = gi.make_device(c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"], c["seed"],
                           device=dev)
        q, k, v, g, b = (d[x] for x in ("q", "k", "v", "g", "beta"))
    o = torch.empty((d["B"], d["T"], d["Hv"], d["dv"]), dtype=torch.bfloat16, device=dev)
    ht = torch.empty((d["B"], d["Hv"], d["dk"], d["dv"]), dtype=torch.float32, device=dev)
    for i in range(n):
        gdn.gdn_chunk_fwd(q, k, v, g, b, out=o, final_state=ht)
        torch.cuda.synchronize()
        print(f"[launch] {i + 1}/{n}", flush=True)
    _calibration_copy(torch, dev)


def _calibration_copy(torch, dev):
    src = torch.zeros(CAL_BYTES // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    print("[launch] calibration copy done", flush=True)


def read_counter(dirname, counter):
    """{kernel name: [value per dispatch]} for one counter."""
    files = glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {dirname}")
    per = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter:
                    continue
                per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return per


def pick(per, needle):
    hits = [(k, v) for k, v in per.items() if needle in k]
    if len(hits) != 1:
        raise SystemExit(f"expected one kernel matching {needle!r}, found {[k for k, _ in hits]}")
    return hits[0]


def traffic_bwd(fetch_dir, write_dir, command, workload):
    """FETCH_SIZE and WRITE_SIZE of each backward kernel, scaled as for the
    forward, against the backward's algorithmic bytes."""
    import gdn_inputs as gi
    c = gi.CONFIGS[workload]
    alg = bench.bwd_algorithmic_bytes(c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"])
    names = [k.format(dk=c["dk"]) for k in BWD_KERNELS]
    fetch, write = read_counter(fetch_dir, "FETCH_SIZE"), read_counter(write_dir, "WRITE_SIZE")
    scale = {}
    for counter, per in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
        _, cv = pick(per, CAL_KERNEL)
        scale[counter] = CAL_BYTES / (sum(cv) / len(cv) * 1024.0)
    rows, total = [], 0.0
    for kname in names:
        r = {"kernel": kname}
        for counter, per in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write)):
            _, kv = pick(per, kname)
            r[counter] = sum(kv) / len(kv) * 1024.0 * scale[counter]
        total += r["FETCH_SIZE"] + r["WRITE_SIZE"]
        rows.append(r)
    out = {"workload": workload,
           "kernel_source_sha256": bench.kernel_source_hash(bench.BWD_KERNEL_SOURCES),
           "algorithmic_bytes_per_call": alg, "scale_factors": scale, "kernels": rows,
           "bytes_per_call": total, "traffic_over_algorithmic": total / alg,
           "command": command}
    with open(os.path.join(PROFILES, f"traffic_{workload}.json"), "w") as f:
        json.dump(out, f, indent=1)
    lines = [f"# HBM traffic of the backward, {workload} (B={c['B']} T={c['T']} H={c['Hv']} "
             f"dk={c['dk']} dv={c['dv']} bf16)", "", "Commands:", "", "```", command, "```", "",
             "FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the same counter reads "
             f"for a copy of 256 MiB (factors {scale['FETCH_SIZE']:.4f} and "
             f"{scale['WRITE_SIZE']:.4f}).", "",
             "| kernel | fetched MB | written MB |", "|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['kernel']}` | {r['FETCH_SIZE'] / 1e6:.1f} | "
                     f"{r['WRITE_SIZE'] / 1e6:.1f} |")
    lines += ["", f"Total {total / 1e6:.1f} MB per call; algorithmic {alg / 1e6:.1f} MB; ratio "
                  f"{total / alg:.3f}.", f"Kernel source sha256 {out['kernel_source_sha256']}."]
    with open(os.path.join(PROFILES, f"traffic_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic(fetch_dir, write_dir, command, workload):
    if workload.startswith("fwd_bwd"):
        return traffic_bwd(fetch_dir, write_dir, command, workload)
    import gdn_inputs as gi
    c = gi.CONFIGS[workload]
    kernel = KERNELS[workload]
    alg = bench.algorithmic_bytes(c["B"], c["T"], c["Hqk"], c["Hv"], c["dk"], c["dv"])
    out = {"kernel": kernel, "workload": workload,
           "kernel_source_sha256": bench.kernel_source_hash(),
           "algorithmic_bytes_per_launch": alg,
           "calibration": f"torch.bitwise_not, int32, {CAL_BYTES} bytes read and {CAL_BYTES} written",
           "command": command}
    total = 0.0
    for counter, dirname in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = read_counter(dirname, counter)
        kname, kv = pick(per, kernel)
        cname, cv = pick(per, CAL_KERNEL)
        cal_kib = sum(cv) / len(cv)
        factor = CAL_BYTES / (cal_kib * 1024.0)
        kib = sum(kv) / len(kv)
        b = kib * 1024.0 * factor
        out[counter] = {"kernel_kib_per_dispatch": kib, "dispatches": len(kv),
                        "calibration_kib": cal_kib, "scale_factor": factor, "bytes": b}
        total += b
    out["bytes_per_launch"] = total
    out["traffic_over_algorithmic"] = total / alg
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"traffic_{workload}.json"), "w") as f:
        json.dump(out, f, indent=1)
    lines = [f"# HBM traffic of {kernel}, {workload} (B={c['B']} T={c['T']} H={c['Hv']} "
             f"dk={c['dk']} dv={c['dv']} bf16)",
             "", "Commands:", "", "```", command, "```", "",
             "| counter | kernel KiB/dispatch | copy KiB (256 MiB known) | scale | bytes/launch |",
             "|---|---|---|---|---|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        r = out[c]
        lines.append(f"| {c} | {r['kernel_kib_per_dispatch']:.0f} | {r['calibration_kib']:.0f} | "
                     f"{r['scale_factor']:.4f} | {r['bytes']:.0f} |")
    lines += ["", f"Total {total:.0f} B per launch; algorithmic {alg} B; ratio "
                  f"{total / alg:.3f}.", f"Kernel source sha256 {out['kernel_source_sha256']}."]
    with open(os.path.join(PROFILES, f"traffic_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


COUNTERS = ["SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_LDS_IDX_ACTIVE",
            "SQ_LDS_BANK_CONFLICT", "SQ_WAVES", "GRBM_GUI_ACTIVE"]


def counters(dirname, command, workload):
    """Writes profiles/counters_W.md from one `rocprofv3 --pmc` run of
    `launch`: each counter averaged over the kernel's dispatches, with the
    ratios the design notes quote.  SQ_VALU_MFMA_BUSY_CYCLES and the LDS
    counters are summed over the chip; GRBM_GUI_ACTIVE is the GPU's busy
    clock count over the dispatch."""
    kernel = KERNELS[workload]
    vals = {}
    for c in COUNTERS:
        per = read_counter(dirname, c)
        kname, kv = pick(per, kernel)
        vals[c] = sum(kv) / len(kv)
    # GRBM_GUI_ACTIVE reads the sum over the 8 XCDs (each has its own
    # GRBM): one XCD's busy clocks are an eighth of it.  MFMA busy cycles
    # are summed over the 1024 SIMDs.
    xcds, simds = 8, 1024
    clocks = vals["GRBM_GUI_ACTIVE"] / xcds
    mfma_util = vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (clocks * simds)
    conflict = vals["SQ_LDS_BANK_CONFLICT"] / max(vals["SQ_LDS_IDX_ACTIVE"], 1.0)
    sources = bench.BWD_KERNEL_SOURCES if workload.startswith("fwd_bwd") else None
    out = {"kernel": kernel, "workload": workload, "command": command,
           "kernel_source_sha256": bench.kernel_source_hash(sources), "per_dispatch": vals,
           "busy_clocks_per_xcd": clocks,
           "mfma_busy_per_simd": mfma_util,
           "lds_bank_conflict_over_idx_active": conflict}
    with open(os.path.join(PROFILES, f"counters_{workload}.json"), "w") as f:
        json.dump(out, f, indent=1)
    lines = [f"# SQ counters of {kernel}, {workload}", "", "Command:", "", "```", command, "```",
             "", "| counter | per dispatch (average) |", "|---|---|"]
    for c in COUNTERS:
        lines.append(f"| {c} | {vals[c]:.4g} |")
    lines += ["",
              f"- GRBM_GUI_ACTIVE sums the 8 XCDs' busy clocks: {clocks:.4g} clocks per XCD "
              f"per dispatch ({clocks / 2.4e3:.1f} us at 2.4 GHz).",
              f"- MFMA busy per SIMD: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 "
              f"SIMDs) = {mfma_util:.3f}.",
              f"- SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE = {conflict:.3f}.",
              f"- Kernel source sha256 {out['kernel_source_sha256']}."]
    with open(os.path.join(PROFILES, f"counters_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


ISSUE_COUNTERS = [
    ["SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
     "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_VALU_MFMA_BUSY_CYCLES",
     "GRBM_GUI_ACTIVE"],
    ["SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
     "SQ_WAIT_INST_LDS", "SQ_LDS_CMD_FIFO_FULL", "SQ_LDS_DATA_FIFO_FULL", "SQ_WAVES",
     "GRBM_GUI_ACTIVE"],
]


def issue(dir_a, dir_b, command, workload):
    """Writes profiles/counters_issue_W.md from two `rocprofv3 --pmc` runs of
    `launch` with the two lists in ISSUE_COUNTERS: how the waves spend their
    cycles (executing VALU or LDS instructions, waiting to issue, waiting for
    anything) as fractions of SQ_WAVE_CYCLES (all four in quad-cycles, summed
    over the waves), and instruction counts per wave and dispatch."""
    kernel = KERNELS[workload]
    vals = {}
    for d, names in ((dir_a, ISSUE_COUNTERS[0]), (dir_b, ISSUE_COUNTERS[1])):
        for c in names:
            per = read_counter(d, c)
            _, kv = pick(per, kernel)
            vals[c if c not in vals else c + " (2nd run)"] = sum(kv) / len(kv)
    wc = vals["SQ_WAVE_CYCLES"]
    waves = vals["SQ_WAVES"]
    clocks = vals["GRBM_GUI_ACTIVE"] / 8
    frac = {k: vals[k] / wc for k in ("SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                                      "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY")}
    per_wave = {k: vals[k] / waves for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS")}
    sources = bench.BWD_KERNEL_SOURCES if workload.startswith("fwd_bwd") else None
    out = {"kernel": kernel, "workload": workload, "command": command,
           "kernel_source_sha256": bench.kernel_source_hash(sources), "per_dispatch": vals,
           "fraction_of_wave_cycles": frac, "instructions_per_wave": per_wave,
           "mfma_busy_per_simd": vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (clocks * 1024),
           "valu_mfma_coexec_per_simd": vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / (clocks * 1024)}
    with open(os.path.join(PROFILES, f"counters_issue_{workload}.json"), "w") as f:
        json.dump(out, f, indent=1)
    lines = [f"# Issue and wait counters of {kernel}, {workload}", "", "Commands:", "", "```",
             command, "```", "", "| counter | per dispatch (average) |", "|---|---|"]
    for c, v in vals.items():
        lines.append(f"| {c} | {v:.4g} |")
    lines += ["", "Fractions of SQ_WAVE_CYCLES (the waves' lifetimes; two waves share each SIMD):", ""]
    for k, v in frac.items():
        lines.append(f"- {k}: {v:.3f}")
    lines += ["", "Per wave and dispatch: " + ", ".join(f"{k} {v:.0f}" for k, v in per_wave.items()) + ".",
              f"MFMA busy per SIMD {out['mfma_busy_per_simd']:.3f}; MFMA and another VALU "
              f"instruction together {out['valu_mfma_coexec_per_simd']:.3f} of each SIMD's clocks "
              f"(both over GRBM_GUI_ACTIVE / 8 x 1024 SIMDs).",
              f"Kernel source sha256 {out['kernel_source_sha256']}."]
    with open(os.path.join(PROFILES, f"counters_issue_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_rows(dirname):
    """Rows like the stats CSV's, one per (kernel, grid size), from the trace."""
    files = glob.glob(os.path.join(dirname, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {dirname}")
    groups = {}
    with open(files[0], newline="") as f:
        for r in csv.DictReader(f):
            grid = "x".join(str(int(r[f"Grid_Size_{a}"]) // int(r[f"Workgroup_Size_{a}"]))
                            for a in "XYZ")
            key = (r["Kernel_Name"], grid)
            groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    total = sum(sum(v) for v in groups.values())
    rows = []
    for (kname, grid), v in groups.items():
        rows.append({"Name": f"{kname} [grid {grid}]", "Calls": len(v),
                     "AverageNs": sum(v) / len(v), "MinNs": min(v), "MaxNs": max(v),
                     "Percentage": 100.0 * sum(v) / total, "TotalNs": sum(v)})
    rows.sort(key=lambda r: -r["TotalNs"])
    return rows


def stats(dirname, command, name="headline_bf16", title=None, only=(), by_grid=False):
    if by_grid:
        rows = trace_rows(dirname)
    else:
        files = glob.glob(os.path.join(dirname, "**", "*kernel_stats.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no kernel_stats.csv under {dirname}")
        with open(files[0], newline="") as f:
            rows = list(csv.DictReader(f))
    if only:
        rows = [r for r in rows if any(s in r["Name"] for s in only)]
    title = title or f"{name}: B=8 T=2048 H=16 d=128 bf16"
    lines = [f"# Kernel time, bench.py ({title})",
             "", "Command:", "", "```", command, "```", ""]
    if only:
        lines += [f"Kernels whose names contain {', '.join(repr(s) for s in only)}; "
                  "the percentages are of the whole run's GPU time.", ""]
    lines += ["| kernel | calls | average µs | min µs | max µs | % of GPU time |",
              "|---|---|---|---|---|---|"]
    for r in rows:
        kname = r["Name"]
        if by_grid:  # keep the template arguments and the grid tag visible
            base, tag = kname.rsplit(" [grid ", 1)
            base = base.replace("void ", "").replace("gdn::(anonymous namespace)::", "")
            short = (base if len(base) <= 60 else base[:57] + "...") + " [grid " + tag
        else:
            short = kname if len(kname) <= 70 else kname[:67] + "..."
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    with open(os.path.join(PROFILES, f"kernel_stats_{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("launch")
    a.add_argument("--launches", type=int, default=5)
    a.add_argument("--workload", default="headline_bf16", choices=sorted(KERNELS))
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--command", required=True)
    t.add_argument("--workload", default="headline_bf16", choices=sorted(KERNELS))
    c = sub.add_parser("counters")
    c.add_argument("pmc_dir")
    c.add_argument("--command", required=True)
    c.add_argument("--workload", default="headline_bf16", choices=sorted(KERNELS))
    i = sub.add_parser("issue")
    i.add_argument("dir_a")
    i.add_argument("dir_b")
    i.add_argument("--command", required=True)
    i.add_argument("--workload", default="headline_bf16", choices=sorted(KERNELS))
    s = sub.add_parser("stats")
    s.add_argument("stats_dir")
    s.add_argument("--command", required=True)
    s.add_argument("--name", default="headline_bf16")
    s.add_argument("--title", default=None)
    s.add_argument("--only", action="append", default=[],
                   help="keep kernels whose name contains this (repeatable)")
    s.add_argument("--by-grid", action="store_true",
                   help="one line per kernel and grid size, from the per-dispatch trace")
    args = ap.parse_args()
    if args.cmd == "launch":
        launch(args.launches, args.workload)
    elif args.cmd == "traffic":
        traffic(args.fetch_dir, args.write_dir, args.command, args.workload)
    elif args.cmd == "counters":
        counters(args.pmc_dir, args.command, args.workload)
    elif args.cmd == "issue":
        issue(args.dir_a, args.dir_b, args.command, args.workload)
    else:
        stats(args.stats_dir, args.command, args.name, args.title, args.only, args.by_grid)


if __name__ == "__main__":
    main()
