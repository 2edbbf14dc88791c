"""Summaries of rocprofv3 output for the kernels of the round.

    python -m chunk_causal_dit_amd.profiling stats  <run_kernel_stats.csv> --cmd "<command>" --out <file.md>
    python -m chunk_causal_dit_amd.profiling traffic --fetch <fetch counter_collection.csv>
        --write <write counter_collection.csv> --kernel <name substring> [--kernel <another> ...]
        --copy-bytes <bytes>
        --cmd "<command>" --source <kernel .hip file> --out <file.json>

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
    the board power sensor; returns mean watts (first quarter of the samples dropped as
    ramp-up), calls made and wall seconds, or None when no sensor is readable."""
    paths = hwmon_power_paths()
    if not paths:
        return None
    path = paths[0]
    samples: List[float] = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                samples.append(float(open(path).read()) * 1e-6)
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
    return {"watts": sum(kept) / len(kept), "calls": calls, "seconds": wall, "sensor": path}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--title", default="rocprofv3 --kernel-trace --stats")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, action="append")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--algorithmic-bytes", type=float, default=None)
    t.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.what == "stats":
        text = f"# {a.title}\n\n" + stats_markdown(a.csv, a.cmd)
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
