"""Summaries of rocprofv3 output for the kernels of the round.

    python -m chunk_causal_dit_amd.profiling stats  <run_kernel_stats.csv> --cmd "<command>" --out <file.md>
    python -m chunk_causal_dit_amd.profiling traffic --fetch <fetch counter_collection.csv>
        --write <write counter_collection.csv> --kernel <name substring> [--kernel <another> ...]
        --copy-bytes <bytes>
        --cmd "<command>" --source <kernel .hip file> --out <file.json>
    python -m chunk_causal_dit_amd.profiling counters <pmc run dir> [<another pass> ...]
        --kernel <name substring> --cmd "<command>" --title "<title>" --out <file.md>

``stats`` turns a ``--kernel-trace --stats`` run into a short markdown table
(calls, average / min / max duration per kernel). ``traffic`` turns two
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs into HBM bytes per launch of
one kernel, or per call of a group of kernels launched once each per call (the
per-kernel figures are kept, and their sum is the call's). Both counters are read in KiB per dispatch; each is calibrated by
what it reads for a plain device-to-device copy of known size in the same run
(the largest dispatch whose name contains "copy"): factor = counter KiB * 1024
/ copy bytes, and the kernel's bytes = counter KiB * 1024 / factor. The JSON
records the sha256 prefix of the kernel source, so a reader can tell when the
counters no longer describe the current kernel.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import threading
import time
from typing import Callable, Dict, List, Optional


def _rows(path: str) -> List[dict]:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def short_name(name: str, width: int = 90) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name if len(name) <= width else name[:width - 3] + "..."


def stats_markdown(stats_csv: str, cmd: str, top: int = 12) -> str:
    rows = _rows(stats_csv)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"Command: `{cmd}`", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def _per_dispatch(path: str, counter: str) -> Dict[int, dict]:
    """dispatch id -> {name, value (summed over the counter's instances), grid}."""
    per: Dict[int, dict] = {}
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        rec = per.setdefault(d, {"name": r["Kernel_Name"], "value": 0.0, "grid": int(r["Grid_Size"])})
        rec["value"] += float(r["Counter_Value"])
    return per


def calibrated_bytes(path: str, counter: str, kernel: str, copy_bytes: int):
    per = _per_dispatch(path, counter)
    copies = [d for d in per.values() if "copy" in d["name"].lower()]
    if not copies:
        raise SystemExit(f"{path}: no copy dispatch to calibrate {counter}")
    ref = max(copies, key=lambda d: d["value"])
    factor = ref["value"] * 1024.0 / copy_bytes
    vals = [d["value"] for d in per.values() if kernel in d["name"]]
    if not vals:
        raise SystemExit(f"{path}: no dispatch of {kernel}")
    kib = sum(vals) / len(vals)
    return {"counter_kib_per_launch": kib, "launches": len(vals), "copy_counter_kib": ref["value"],
            "factor": factor, "bytes_per_launch": kib * 1024.0 / factor}


def hwmon_power_paths() -> List[str]:
    """Board power sensors (microwatts) of the GPUs visible under /sys/class/drm."""
    paths = []
    for h in sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*")):
        for name in ("power1_average", "power1_input"):
            p = os.path.join(h, name)
            if os.path.exists(p):
                paths.append(p)
                break
    return paths


def sample_power(run: Callable[[], None], sync: Callable[[], None], seconds: float = 3.0,
                 period: float = 0.01) -> Optional[dict]:
    """Calls run() repeatedly for about `seconds` (sync() after each call) while a thread reads
    the board power sensor and, where the same hwmon directory has one, the shader clock
    sensor (freq1_input, Hz); returns mean watts and mean clock in MHz (first quarter of the
    samples dropped as ramp-up), calls made and wall seconds, or None when no power sensor
    is readable."""
    paths = hwmon_power_paths()
    if not paths:
        return None
    path = paths[0]
    # shader clock: hwmon freq1_input (Hz) where the driver has it, else the current
    # level of pp_dpm_sclk (the line marked "*", in MHz) of the same device
    clk_path = os.path.join(os.path.dirname(path), "freq1_input")
    if not os.path.exists(clk_path):
        clk_path = os.path.join(os.path.dirname(os.path.dirname(os.path.dirname(path))), "pp_dpm_sclk")
        if not os.path.exists(clk_path):
            clk_path = None

    def read_clock_mhz() -> Optional[float]:
        text = open(clk_path).read()
        if clk_path.endswith("freq1_input"):
            return float(text) * 1e-6
        for line in text.splitlines():
            if line.rstrip().endswith("*"):
                return float(line.split(":")[1].strip().lower().split("mhz")[0])
        return None
    samples: List[float] = []
    clocks: List[float] = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                samples.append(float(open(path).read()) * 1e-6)
                if clk_path:
                    c = read_clock_mhz()
                    if c is not None:
                        clocks.append(c)
            except (OSError, ValueError):
                pass
            time.sleep(period)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    calls, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        run()
        sync()
        calls += 1
    wall = time.perf_counter() - t0
    stop.set()
    th.join()
    kept = samples[len(samples) // 4:]
    if not kept:
        return None
    ck = clocks[len(clocks) // 4:]
    cap_path = os.path.join(os.path.dirname(path), "power1_cap")
    try:
        cap = float(open(cap_path).read()) * 1e-6
    except (OSError, ValueError):
        cap = None
    return {"watts": sum(kept) / len(kept), "cap_watts": cap, "clock_mhz": (sum(ck) / len(ck)) if ck else None,
            "calls": calls, "seconds": wall, "sensor": path, "clock_sensor": clk_path}


def counters_markdown(runs: List[str], kernel: str, cmd: str, n_simd: int = 1024, skip_first: bool = True,
                      mfma_per_tile: int = 0) -> str:
    """Per-launch counters of one kernel from one or more --pmc runs (directories holding a
    run_counter_collection.csv and run_kernel_trace.csv; each run one pass of counters).
    Values are summed over a dispatch's counter instances, then averaged over the kernel's
    dispatches (the first, a warm-up, dropped when there are more). Derived: the shader
    clock GRBM_GUI_ACTIVE / 8 XCDs / duration; MFMA busy and MFMA/VALU co-execution as
    shares of SIMD-cycles (n_simd SIMDs x clock cycles); instructions per wave; and, when
    the busy, co-execution and SQ_ACTIVE_INST_VALU counters are all present, the split of
    SIMD time into MFMA only, VALU only, both and neither (SQ_ACTIVE_INST_* count 4-cycle
    units). With mfma_per_tile > 0 the instruction counts are also given per key tile and
    wave (MFMA instructions per wave / mfma_per_tile tiles)."""
    merged: Dict[str, float] = {}
    clocks, durs = [], []
    for d in runs:
        per: Dict[int, Dict[str, float]] = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in _rows(glob.glob(os.path.join(d, "*counter_collection.csv"))[0]):
            if kernel in r["Kernel_Name"]:
                per[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        trace = {int(r["Dispatch_Id"]): int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                 for r in _rows(glob.glob(os.path.join(d, "*kernel_trace.csv"))[0])}
        ids = sorted(per)
        if skip_first and len(ids) > 1:
            ids = ids[1:]
        for name in per[ids[0]]:
            merged[name] = sum(per[i][name] for i in ids) / len(ids)
        if "GRBM_GUI_ACTIVE" in per[ids[0]]:
            for i in ids:
                clocks.append(per[i]["GRBM_GUI_ACTIVE"] / 8 / trace[i])
                durs.append(trace[i])
    out = [f"Kernel: `{kernel}`", "", f"Command (one run per pass of counters): `{cmd}`", "",
           "| quantity (per launch, mean over the launches after the first) | value |", "|---|---|"]
    if durs:
        out.append(f"| duration under the profiler | {sum(durs) / len(durs) / 1e3:.1f} us |")
        out.append(f"| shader clock = GRBM_GUI_ACTIVE / 8 / duration | {sum(clocks) / len(clocks):.2f} GHz |")
    cyc = merged.get("GRBM_GUI_ACTIVE", 0.0) / 8
    if cyc and "SQ_VALU_MFMA_BUSY_CYCLES" in merged:
        out.append(f"| MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / ({n_simd} SIMDs x cycles) | "
                   f"{merged['SQ_VALU_MFMA_BUSY_CYCLES'] / n_simd / cyc * 100:.1f} % |")
    if cyc and "SQ_VALU_MFMA_COEXEC_CYCLES" in merged:
        out.append(f"| VALU co-executing with MFMA = SQ_VALU_MFMA_COEXEC_CYCLES / SIMD-cycles | "
                   f"{merged['SQ_VALU_MFMA_COEXEC_CYCLES'] / n_simd / cyc * 100:.1f} % |")
    waves = merged.get("SQ_WAVES")
    for name in sorted(merged):
        if name in ("GRBM_GUI_ACTIVE",):
            continue
        v = merged[name]
        per_wave = f" ({v / waves:.0f} per wave)" if waves and name.startswith("SQ_INSTS") else ""
        out.append(f"| {name} | {v:.4g}{per_wave} |")
    need = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU")
    if cyc and all(n in merged for n in need):
        simd_cyc = n_simd * cyc
        mf = merged["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cyc
        both = merged["SQ_VALU_MFMA_COEXEC_CYCLES"] / simd_cyc
        va = merged["SQ_ACTIVE_INST_VALU"] * 4 / simd_cyc
        out += ["", "| share of SIMD-cycles | value |", "|---|---|",
                f"| MFMA busy | {mf * 100:.1f} % |", f"| VALU issuing (SQ_ACTIVE_INST_VALU x 4) | {va * 100:.1f} % |",
                f"| both at once (SQ_VALU_MFMA_COEXEC_CYCLES) | {both * 100:.1f} % |",
                f"| MFMA only | {(mf - both) * 100:.1f} % |", f"| VALU only | {(va - both) * 100:.1f} % |",
                f"| neither (barrier waits, LDS and SMEM latency, scalar-only issue) | "
                f"{(1 - mf - va + both) * 100:.1f} % |"]
    if mfma_per_tile and waves and "SQ_INSTS_MFMA" in merged:
        tiles = merged["SQ_INSTS_MFMA"] / waves / mfma_per_tile
        rows = [("MFMA", "SQ_INSTS_MFMA"), ("LDS instructions", "SQ_INSTS_LDS"),
                ("VALU instructions (MFMA included)", "SQ_INSTS_VALU"), ("of which v_exp_f32 and other fp32 "
                                                                        "transcendentals", "SQ_INSTS_VALU_TRANS_F32"),
                ("SALU instructions", "SQ_INSTS_SALU")]
        out += ["", f"Per 64-key tile and wave ({tiles:.0f} tiles per wave = MFMA per wave / {mfma_per_tile}):", "",
                "| instructions | per tile and wave |", "|---|---|"]
        for label, name in rows:
            if name in merged:
                out.append(f"| {label} | {merged[name] / waves / tiles:.1f} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", default="rocprofv3 --kernel-trace --stats")
    s.add_argument("--note", default="", help="text appended after the table")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, action="append")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--algorithmic-bytes", type=float, default=None)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("runs", nargs="+", help="rocprofv3 output directories, one per pass of counters")
    c.add_argument("--kernel", required=True)
    c.add_argument("--cmd", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--mfma-per-tile", type=int, default=0, help="MFMA instructions per key tile and wave")
    c.add_argument("--note", default="", help="text appended after the tables")
    a = ap.parse_args(argv)
    if a.what == "counters":
        text = f"# {a.title}\n\n" + counters_markdown(a.runs, a.kernel, a.cmd, mfma_per_tile=a.mfma_per_tile)
        if a.note:
            text += "\n" + a.note.strip() + "\n"
        open(a.out, "w").write(text)
        print(text)
        return
    if a.what == "stats":
        text = f"# {a.title}\n\n" + stats_markdown(a.csv, a.cmd)
        if a.note:
            text += "\n" + a.note.strip() + "\n"
        open(a.out, "w").write(text)
        print(text)
        return
    per_kernel = {}
    for k in a.kernel:
        fetch = calibrated_bytes(a.fetch, "FETCH_SIZE", k, a.copy_bytes)
        write = calibrated_bytes(a.write, "WRITE_SIZE", k, a.copy_bytes)
        per_kernel[k] = {"fetch": fetch, "write": write,
                         "hbm_bytes_per_launch": fetch["bytes_per_launch"] + write["bytes_per_launch"]}
    rec = {
        "kernel": " + ".join(a.kernel),
        "command": a.cmd,
        "kernel_source_sha256_16": hashlib.sha256(open(a.source, "rb").read()).hexdigest()[:16],
        "copy_bytes": a.copy_bytes,
    }
    if len(a.kernel) == 1:
        rec.update({"fetch": per_kernel[a.kernel[0]]["fetch"], "write": per_kernel[a.kernel[0]]["write"]})
    else:
        rec["per_kernel"] = per_kernel
    rec["hbm_bytes_per_launch"] = sum(v["hbm_bytes_per_launch"] for v in per_kernel.values())
    rec["algorithmic_bytes_per_launch"] = a.algorithmic_bytes
    json.dump(rec, open(a.out, "w"), indent=1)
    json.dump(rec, sys.stdout, indent=1)
    print()


if __name__ == "__main__":
    main()
