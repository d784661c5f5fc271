#!/usr/bin/env python3
"""HBM traffic of one attention call from two rocprofv3 counter runs.

bench.py --traffic-probe runs a plain device copy of known size (the
calibration kernel) and a few mla_decode_attn calls.  Run it twice under
rocprofv3 on the GPU, once per counter (the counters go in separate runs):

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- \\
        python3 bench.py --traffic-probe > gpurun_out/pmc_fetch.log
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- \\
        python3 bench.py --traffic-probe > gpurun_out/pmc_write.log

then, anywhere:

    python3 bench_traffic.py gpurun_out/pmc_fetch gpurun_out/pmc_write

FETCH_SIZE / WRITE_SIZE are read in KiB per dispatch.  Each is scaled by the
factor that makes the copy kernel's reading equal its true size (copy bytes
read, resp. written), and the attention call's traffic is the sum over its
kernels (the decode kernels the plan launched, and combine_kernel).
Writes profiles/decode_traffic.json (read by bench.py, which uses it only
when the workload and the kernel sources match) and a short summary.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
ATTN_KERNELS = ("decode_mfma_kernel", "decode_fp8_kernel", "decode_small_kernel", "decode_x2_kernel",
                "decode_general_kernel", "combine_kernel")
COPY_KERNEL = "copyBuffer"


def read_counter(run_dir: str, counter: str):
    """{dispatch_id: (kernel name, value)} for one counter."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    out = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                d = int(row["Dispatch_Id"])
                name, val = row["Kernel_Name"], float(row["Counter_Value"])
                prev = out.get(d, (name, 0.0))
                out[d] = (name, prev[1] + val)       # sum over dimension rows, if any
    return out


def probe_info(run_dir: str):
    log = run_dir.rstrip("/") + ".log"
    with open(log) as f:
        for line in f:
            if line.startswith("{") and "traffic_probe" in line:
                return json.loads(line)
    raise SystemExit(f"no probe line in {log}")


def summarise(run_dir: str, counter: str, copy_bytes: int):
    vals = read_counter(run_dir, counter)
    copies = [v for n, v in vals.values() if COPY_KERNEL in n]
    if not copies:
        raise SystemExit(f"{counter}: no copy dispatch found")
    # the calibration copies are the large ones (small copies are uploads)
    copies = [v for v in copies if v >= 0.5 * max(copies)]
    copy_kib = statistics.median(copies)
    factor = copy_bytes / (copy_kib * 1024.0)
    per_kernel = {}
    for k in ATTN_KERNELS:
        xs = [v for n, v in vals.values() if k in n]
        if xs:
            per_kernel[k] = statistics.median(xs) * 1024.0 * factor
    return {"counter": counter, "copy_kib": copy_kib, "factor": factor,
            "bytes_per_kernel": per_kernel}


def main():
    if len(sys.argv) != 3:
        raise SystemExit(__doc__)
    fetch_dir, write_dir = sys.argv[1], sys.argv[2]
    pf, pw = probe_info(fetch_dir), probe_info(write_dir)
    assert pf["sources_sha256"] == pw["sources_sha256"] and pf["workload"] == pw["workload"]
    fetch = summarise(fetch_dir, "FETCH_SIZE", pf["copy_bytes"])
    write = summarise(write_dir, "WRITE_SIZE", pw["copy_bytes"])
    fb = sum(fetch["bytes_per_kernel"].values())
    wb = sum(write["bytes_per_kernel"].values())
    rec = {
        "workload": pf["workload"],
        "sources_sha256": pf["sources_sha256"],
        "hbm_bytes_per_launch": round(fb + wb),
        "fetch_bytes_per_launch": round(fb),
        "write_bytes_per_launch": round(wb),
        "bytes_alg_per_launch": pf["bytes_alg_per_launch"],
        "fetch": fetch,
        "write": write,
    }
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "decode_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    lines = [f"# HBM traffic of one mla_decode_attn call, workload {rec['workload']}", "",
             "Commands (repo root, MI355X; counters in separate runs):", "",
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- \\",
             "        python3 bench.py --traffic-probe > gpurun_out/pmc_fetch.log",
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- \\",
             "        python3 bench.py --traffic-probe > gpurun_out/pmc_write.log",
             "    python3 bench_traffic.py gpurun_out/pmc_fetch gpurun_out/pmc_write", "",
             "Calibration: a device copy of %d bytes read %.0f KiB (FETCH_SIZE, factor %.4f) "
             "and wrote %.0f KiB (WRITE_SIZE, factor %.4f)." % (
                 pf["copy_bytes"], fetch["copy_kib"], fetch["factor"], write["copy_kib"],
                 write["factor"]), "",
             "| kernel | fetch (MB) | write (MB) |", "|---|---:|---:|"]
    for k in ATTN_KERNELS:
        if k in fetch["bytes_per_kernel"] or k in write["bytes_per_kernel"]:
            lines.append("| %s | %.2f | %.2f |" % (k, fetch["bytes_per_kernel"].get(k, 0) / 1e6,
                                                  write["bytes_per_kernel"].get(k, 0) / 1e6))
    lines += ["", "Per call: %.2f MB fetched + %.2f MB written = %.2f MB; algorithmic bytes "
              "(cache + absorbed queries + latent output + LSE) %.2f MB." % (
                  fb / 1e6, wb / 1e6, (fb + wb) / 1e6, rec["bytes_alg_per_launch"] / 1e6), ""]
    name = f"traffic_{rec['workload']}.md"
    with open(os.path.join(ROOT, "profiles", name), "w") as f:
        f.write("\n".join(lines))
    print(json.dumps({k: rec[k] for k in ("workload", "hbm_bytes_per_launch",
                                          "fetch_bytes_per_launch", "write_bytes_per_launch",
                                          "bytes_alg_per_launch")}))


if __name__ == "__main__":
    main()
