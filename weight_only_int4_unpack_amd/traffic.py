"""HBM traffic of the decode workload from two rocprofv3 counter passes.

Reads the counter CSVs of ``rocprofv3 --pmc FETCH_SIZE`` and of
``rocprofv3 --pmc WRITE_SIZE`` over ``bench.py ... --copy-probe`` (the decode
workload plus one plain 256 MiB device copy) and writes the bytes per launch
that ``bench.py`` reports as ``roofline.traffic``:

* calibration: the copy of 256 MiB (the dispatch that writes 262144 KiB) reads
  and writes 256 MiB; the counters' readings for it give one scale per
  counter (FETCH_SIZE reads half the bytes on this GPU, WRITE_SIZE all);
* each decode kernel instantiation (M = 1 and M = 5 use different row
  counts) is averaged over its dispatches; bytes per launch is the mean of
  (read + write) over the two;
* the record carries the hash of the kernel source it was taken on; bench.py
  reports null once the source changes.

Usage: ``python -m weight_only_int4_unpack_amd.traffic FETCH_DIR WRITE_DIR [OUT]``
(OUT defaults to profiles/traffic.json).
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KIB = 262144.0   # the calibration copy: 256 MiB


def _rows(d: str):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _by_dispatch(rows):
    out = collections.defaultdict(float)
    names = {}
    for r in rows:                      # sum over the counter's instances
        out[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    return out, names


def kernel_sha() -> str:
    src = os.path.join(PKG, "csrc", "w4a16_kernels.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def summarise(fetch_dir: str, write_dir: str) -> dict:
    fetch, names = _by_dispatch(_rows(fetch_dir))
    write, wnames = _by_dispatch(_rows(write_dir))
    # calibration copy: in each pass, the copy dispatch with the largest reading
    cf = max((d for d in fetch if "copyBuffer" in names[d]), key=lambda d: fetch[d])
    cw = max((d for d in write if "copyBuffer" in wnames[d]), key=lambda d: write[d])
    if abs(write[cw] - COPY_KIB) > 1.0:
        raise ValueError(f"no 256 MiB calibration copy in the WRITE_SIZE pass ({write[cw]} KiB)")
    fscale, wscale = COPY_KIB / fetch[cf], COPY_KIB / write[cw]
    groups_f, groups_w = collections.defaultdict(list), collections.defaultdict(list)
    for d, v in fetch.items():
        if "decode_kernel" in names[d]:
            groups_f[names[d]].append(v * fscale * 1024)
    for d, v in write.items():
        if "decode_kernel" in wnames[d]:
            groups_w[wnames[d]].append(v * wscale * 1024)
    per = {}
    for name in sorted(groups_f):
        # template arguments (type, zero points, mode, aligned, steps, rows
        # rounded up, sliding window): rows 4 for M = 1, 8 for M = 5
        targs = [t.strip() for t in name.split("(w4a16::DecodeParams")[0].rsplit("<", 1)[1]
                 .rstrip(">").split(",")]
        rows = {"4": "M=1", "8": "M=5"}[targs[5]]
        per[rows] = {"read": statistics.mean(groups_f[name]),
                     "write": statistics.mean(groups_w[name]), "dispatches": len(groups_f[name])}
    sys.path.insert(0, ROOT)
    import bench                                          # noqa: E402
    from weight_only_int4_unpack_amd import synthetic     # noqa: E402
    alg = {"M=1": bench.alg_bytes(synthetic.WORKLOADS["decode_m1"]),
           "M=5": bench.alg_bytes(synthetic.WORKLOADS["decode_m5"])}
    total = statistics.mean(p["read"] + p["write"] for p in per.values())
    return {"decode_m1+decode_m5": {
        "bytes_per_launch": int(round(total)),
        "read_bytes": {k: int(round(v["read"])) for k, v in per.items()},
        "write_bytes": {k: int(round(v["write"])) for k, v in per.items()},
        "algorithmic_bytes": alg,
        "calibration": {"fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
                        "by": "a 256 MiB device-to-device copy in the same run, read with the "
                              "same counters"},
        "note": "above the algorithmic bytes: the fp32 split-K partials (splits x M x N x 4 B) "
                "written and read back once",
        "kernel_sha": kernel_sha(),
        "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <dir> -o "
                   "bench -- python3 bench.py --steps 10 --warmup 2 --no-cpu --no-prefill-extra "
                   "--no-context --copy-probe; python -m weight_only_int4_unpack_amd.traffic "
                   "<fetch dir> <write dir>"}}


def main(argv):
    if len(argv) < 2:
        print(__doc__)
        return 2
    out = argv[2] if len(argv) > 2 else os.path.join(ROOT, "profiles", "traffic.json")
    rec = summarise(argv[0], argv[1])
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
