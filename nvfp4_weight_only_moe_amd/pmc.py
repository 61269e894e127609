"""HBM traffic per kernel launch from rocprofv3 counter runs.

rocprofv3 ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (one counter per run)
write ``*_counter_collection.csv`` files with one row per dispatch and the
counter in KiB.  The counters are scaled by what they read for a plain device
copy of known size in the same run (``bench.py --copy-calibration``: the last
three ``__amd_rocclr_copyBuffer`` dispatches copy 268,435,456 bytes each), so
that the figure is in bytes of HBM traffic whatever unit the counter really
counts.  The result goes into ``profiles/traffic.json``, keyed
``<kernel>@<workload>`` and stamped with the hash of the kernel's sources, and
``bench.py`` reports it as ``roofline.traffic`` while the hash still matches.

    python -m nvfp4_weight_only_moe_amd.pmc --fetch DIR --write DIR \\
        --workload NAME --kernel SHORT=REGEX [--kernel ...] [--update traffic.json]

prints one markdown row per kernel (dispatches, read and written bytes per
launch) and, with ``--update``, merges the entries into the JSON file.
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
CALIBRATION_BYTES = 268435456
CALIBRATION_COPIES = 3

# Sources that determine each kernel's memory traffic; the stored counters
# are valid while these files are unchanged.
KERNEL_SOURCES = {
    "dec_gateup": ["moe_decode.hip", "device_common.h", "route_common.h", "quant_common.h"],
    "dec_gateup_route": ["moe_decode.hip", "device_common.h", "route_common.h", "quant_common.h"],
    "dec_down": ["moe_decode.hip", "device_common.h", "route_common.h", "quant_common.h"],
    "gemm_gateup": ["moe_prefill.hip", "moe_prefill_pipe.hip", "device_common.h"],
    "gemm_down": ["moe_prefill.hip", "moe_prefill_pipe.hip", "device_common.h"],
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_dispatches(directory, counter):
    """[(dispatch_id, kernel_name, value_kib)] for one counter, every CSV under directory."""
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)):
        with open(path, newline="") as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


def copy_scale(rows):
    """Bytes per counter KiB, from the calibration copies (the last copies of the run)."""
    copies = [v for _, name, v in rows if "copyBuffer" in name]
    if len(copies) < CALIBRATION_COPIES:
        raise SystemExit("no calibration copies in the run: pass --copy-calibration to bench.py")
    cal = copies[-CALIBRATION_COPIES:]
    mean_kib = sum(cal) / len(cal)
    return CALIBRATION_BYTES / (mean_kib * 1024.0)


def per_launch(rows, regex, scale):
    vals = [v for _, name, v in rows if re.search(regex, name)]
    if not vals:
        return 0, None
    return len(vals), sum(vals) / len(vals) * 1024.0 * scale


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--fetch", required=True, help="directory of the FETCH_SIZE run")
    ap.add_argument("--write", required=True, help="directory of the WRITE_SIZE run")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--kernel", action="append", required=True, metavar="SHORT=REGEX")
    ap.add_argument("--update", help="traffic JSON file to merge the entries into")
    args = ap.parse_args(argv)

    fetch = read_dispatches(args.fetch, "FETCH_SIZE")
    write = read_dispatches(args.write, "WRITE_SIZE")
    sf, sw = copy_scale(fetch), copy_scale(write)
    print(f"copy calibration: FETCH_SIZE scale {sf:.4f}, WRITE_SIZE scale {sw:.4f} (bytes per counted byte)")
    print("| kernel | dispatches | HBM read B | HBM write B |")
    print("|---|---|---|---|")
    entries = {}
    for spec in args.kernel:
        short, regex = spec.split("=", 1)
        nf, rb = per_launch(fetch, regex, sf)
        nw, wb = per_launch(write, regex, sw)
        if rb is None or wb is None:
            print(f"| `{short}` | no dispatch matched {regex!r} | | |")
            continue
        print(f"| `{short}` | {nf} | {rb:,.0f} | {wb:,.0f} |")
        entries[f"{short}@{args.workload}"] = {
            "hbm_bytes_per_launch": int(round(rb + wb)),
            "fetch_bytes": int(round(rb)),
            "write_bytes": int(round(wb)),
            "source_sha256": kernel_source_hash(short),
            "copy_scale_fetch": round(sf, 4),
            "copy_scale_write": round(sw, 4),
        }
    if args.update:
        data = {}
        if os.path.exists(args.update):
            with open(args.update) as fh:
                data = json.load(fh)
        data.update(entries)
        with open(args.update, "w") as fh:
            json.dump(data, fh, indent=1, sort_keys=True)
            fh.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
