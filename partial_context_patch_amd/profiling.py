"""Summaries of rocprofv3 output for the kernels of this library.

    python -m partial_context_patch_amd.profiling stats <trace_dir> --workload W --cmd "..."
    python -m partial_context_patch_amd.profiling counters <pmc_dir> [<pmc_dir> ...] --workload W --cmd "..."

`stats` reads <trace_dir>/*kernel_stats.csv (rocprofv3 --kernel-trace --stats
--output-format csv).  `counters` reads <pmc_dir>/*counter_collection.csv of
one or more --pmc passes over a bench.py run made with --copy-calibration:
the plain 512 MiB copy in that run scales FETCH_SIZE and WRITE_SIZE (KiB per
dispatch) to bytes.  Both print a short text summary; the counters summary
ends with one `summary-json:` line that bench.py reads for roofline.traffic,
valid only while the kernel source hash it records still matches.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
from collections import defaultdict
from typing import Dict, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ("csrc/attn_bf16.hip", "csrc/npa_internal.hpp", "csrc/api.cpp")
COPY_BYTES = 512 << 20


def _code_only(text: str) -> str:
    """The source with // comments, trailing blanks and blank lines removed, so
    that an edit to comments alone keeps the hash (string literals in these
    kernel sources hold no //)."""
    lines = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            lines.append(code)
    return "\n".join(lines)


def kernel_source_hash(sources: Optional[Dict[str, str]] = None) -> str:
    """Hash of the attention kernel's code (comments excluded) -- a counter
    summary applies only to the code it was taken on.  `sources` maps the
    KERNEL_SOURCES paths to their text (default: the files on disk)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if sources is not None:
            text = sources[rel]
        else:
            with open(os.path.join(HERE, rel), encoding="utf-8") as f:
                text = f.read()
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("npa::(anonymous namespace)::", "")
    return name.split("(")[0] if "npa" in name or "attn" in name or "sg_blend" in name else name[:60]


def stats(trace_dir: str, workload: str, cmd: str) -> str:
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(files[0])))
    out = [f"rocprofv3 kernel trace summary -- workload {workload}",
           f"command (from the repository root): {cmd}",
           "",
           f"{'kernel':64s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share':>7s}"]
    for r in rows:
        out.append(f"{_short(r['Name']):64s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}%")
    return "\n".join(out) + "\n"


def counters(pmc_dirs, workload: str, cmd: str) -> str:
    per: Dict[str, Dict[str, list]] = defaultdict(lambda: defaultdict(list))
    for d in pmc_dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                per[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    copy = next((k for k in per if "copyBuffer" in k), None)
    attn = next((k for k in per if "attn_bf16_kernel" in k or "attn_f32_kernel" in k), None)
    sg = next((k for k in per if "sg_blend" in k), None)
    if attn is None:
        raise SystemExit("need the attention kernel in the counter runs")
    mean = lambda k, c: statistics.fmean(per[k][c]) if per[k].get(c) else None
    f_fetch = f_write = None
    if copy is not None:
        f_fetch = COPY_BYTES / (mean(copy, "FETCH_SIZE") * 1024) if mean(copy, "FETCH_SIZE") else None
        f_write = COPY_BYTES / (mean(copy, "WRITE_SIZE") * 1024) if mean(copy, "WRITE_SIZE") else None
    fmt = lambda f: "n/a" if f is None else f"x{f:.3f}"
    lines = [f"rocprofv3 counter summary -- workload {workload}",
             f"commands (from the repository root), one run per pass: {cmd}",
             f"kernel source hash: {kernel_source_hash()}",
             (f"calibration copy ({COPY_BYTES >> 20} MiB read + written): FETCH_SIZE {fmt(f_fetch)}, "
              f"WRITE_SIZE {fmt(f_write)}") if copy is not None else "no calibration copy in these runs",
             ""]
    summary = {"workload": workload, "kernel_source_hash": kernel_source_hash(),
               "fetch_scale": f_fetch, "write_scale": f_write}
    for key, k in (("attention", attn), ("sg_blend", sg)):
        if k is None:
            continue
        lines.append(f"{_short(k)}  (mean per dispatch)")
        for c in sorted(per[k]):
            lines.append(f"    {c:30s} {mean(k, c):16.6g}")
        fetch = mean(k, "FETCH_SIZE")
        write = mean(k, "WRITE_SIZE")
        if fetch is not None and write is not None and f_fetch and f_write:
            hbm = fetch * 1024 * f_fetch + write * 1024 * f_write
            lines.append(f"    -> HBM bytes per dispatch (scaled): read {fetch * 1024 * f_fetch / 1e6:.1f} MB, "
                         f"write {write * 1024 * f_write / 1e6:.1f} MB, total {hbm / 1e6:.1f} MB")
            summary[f"{key}_hbm_bytes"] = hbm
        busy = mean(k, "SQ_VALU_MFMA_BUSY_CYCLES")
        gui = mean(k, "GRBM_GUI_ACTIVE")
        if busy is not None and gui:
            lines.append(f"    -> MFMA busy per SIMD: {busy / 1024 / (gui / 8) * 100:.1f}% of the kernel's cycles "
                         f"(GRBM_GUI_ACTIVE summed over 8 XCDs)")
        conf, act = mean(k, "SQ_LDS_BANK_CONFLICT"), mean(k, "SQ_LDS_IDX_ACTIVE")
        if conf is not None and act:
            lines.append(f"    -> LDS bank-conflict cycles: {100 * conf / act:.1f}% of LDS-active cycles")
        lines.append("")
    lines.append("summary-json: " + json.dumps(summary))
    return "\n".join(lines) + "\n"


def load_traffic(workload: str) -> Optional[float]:
    """HBM bytes per attention dispatch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"attn_bf16_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("summary-json: "):
            s = json.loads(line[len("summary-json: "):])
            if s.get("kernel_source_hash") == kernel_source_hash():
                return s.get("attention_hbm_bytes")
    return None


class ClockSampler:
    """Samples the GPU's current shader clock (the starred level of
    pp_dpm_sclk, in MHz) and board power (hwmon power1_input, in W) from sysfs
    on a background thread, every `period` seconds, between start() and stop().
    Reads only; when the files are absent the results are None."""

    def __init__(self, period: float = 0.002):
        import threading
        self.period = period
        self.sclk, self.power = [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        dev = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self._sclk_path = dev[0] if dev else None
        hw = sorted(glob.glob(os.path.join(os.path.dirname(dev[0]), "hwmon", "hwmon*", "power1_input"))) if dev else []
        self._power_path = hw[0] if hw else None
        cap = os.path.join(os.path.dirname(hw[0]), "power1_cap") if hw else None
        self.power_cap_w = None
        if cap and os.path.exists(cap):
            try:
                self.power_cap_w = int(open(cap).read()) / 1e6
            except (OSError, ValueError):
                pass

    def _run(self):
        import time
        while not self._stop.is_set():
            try:
                if self._sclk_path:
                    for line in open(self._sclk_path):
                        if line.rstrip().endswith("*"):
                            self.sclk.append(float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0]))
                if self._power_path:
                    self.power.append(int(open(self._power_path).read()) / 1e6)
            except (OSError, ValueError, IndexError):
                pass
            time.sleep(self.period)

    def start(self):
        self._thread.start()
        return self

    def stop(self):
        self._stop.set()
        self._thread.join()

    def summary(self) -> dict:
        mean = lambda v: round(statistics.fmean(v), 1) if v else None
        return {"sclk_mhz": mean(self.sclk), "sclk_samples": len(self.sclk), "power_w": mean(self.power),
                "power_cap_w": self.power_cap_w}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    b = sub.add_parser("counters")
    b.add_argument("dirs", nargs="+")
    for p in (a, b):
        p.add_argument("--workload", required=True)
        p.add_argument("--cmd", required=True)
    args = ap.parse_args(argv)
    if args.what == "stats":
        sys.stdout.write(stats(args.dir, args.workload, args.cmd))
    else:
        sys.stdout.write(counters(args.dirs, args.workload, args.cmd))
    return 0


if __name__ == "__main__":
    sys.exit(main())
