"""Per-launch HBM traffic from rocprofv3 counter dumps, for bench.py (measurement
tooling beside the benchmark, not part of the q3 library).

    python bench_traffic.py FETCH.csv WRITE.csv > profiles/traffic.json

FETCH.csv / WRITE.csv are the `*_counter_collection.csv` files of two
`rocprofv3 --pmc FETCH_SIZE` and `rocprofv3 --pmc WRITE_SIZE` runs of a
`bench.py ... --calibrate-copy` command.  Each counter is scaled by what it reads
for the plain 256 MiB device-to-device copy in the same run (known bytes read
and written), which corrects for the share of the memory system the counter
block observes.  Several runs may be merged (pairs of files, in order).  The
result is keyed by a hash of the library sources, so bench.py ignores it as
soon as a kernel changes.
"""
from __future__ import annotations

import collections
import csv
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "bit_fp8_codebook_amd", "csrc")
COPY_BYTES = 256 << 20


def source_hash() -> str:
    """Hash of the library's kernel and ABI sources (names and contents)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def per_kernel(path, counter):
    vals = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


KEYS = ("splitk_full_kernel<", "splitk_kernel<", "linear_kernel<", "wide_hs_kernel<", "wide_kernel<",
        "split_reduce_kernel<", "fit_kernel", "pack_kernel", "unpack_kernel",
        "budget_topk_wave_kernel<", "topk_wave_kernel", "budget_topk_kernel", "topk_kernel", "combine_kernel",
        "quantize_kernel", "shortlist_chunks", "rescore_kernel", "read_kernel<", "copyBuffer")


def short(name: str) -> str:
    """Kernel name without namespaces and argument lists (template arguments kept)."""
    for key in KEYS:
        if key in name:
            i = name.index(key)
            if key.endswith("<") and ">" in name[i:]:
                return name[i:name.index(">", i) + 1]
            return key
    return name[:60]


def merge(pairs):
    """[(fetch_csv, write_csv), ...] -> the traffic.json dict."""
    out = {"source_hash": source_hash(), "runs": [], "kernels": {}}
    acc = collections.defaultdict(lambda: {"read": [], "write": []})
    for fetch_csv, write_csv in pairs:
        f = per_kernel(fetch_csv, "FETCH_SIZE")
        w = per_kernel(write_csv, "WRITE_SIZE")
        copy_f = [v for k, vs in f.items() if "copyBuffer" in k for v in vs]
        copy_w = [v for k, vs in w.items() if "copyBuffer" in k for v in vs]
        if not copy_f or not copy_w:
            raise SystemExit(f"{fetch_csv} / {write_csv}: no calibration copy (run bench.py with --calibrate-copy)")
        # the calibration copy is the largest copy in the run
        fs = COPY_BYTES / 1024 / max(copy_f)
        ws = COPY_BYTES / 1024 / max(copy_w)
        out["runs"].append({"fetch": os.path.basename(os.path.dirname(fetch_csv)), "fetch_scale": fs,
                            "write": os.path.basename(os.path.dirname(write_csv)), "write_scale": ws})
        for k, vs in f.items():
            if "copyBuffer" not in k:
                acc[short(k)]["read"] += [v * 1024 * fs for v in vs]
        for k, vs in w.items():
            if "copyBuffer" not in k:
                acc[short(k)]["write"] += [v * 1024 * ws for v in vs]
    for k, v in acc.items():
        rd, wr = v["read"], v["write"]
        out["kernels"][k] = {"read_bytes": round(sum(rd) / len(rd)) if rd else None,
                             "write_bytes": round(sum(wr) / len(wr)) if wr else None,
                             "dispatches": len(rd)}
    return out


def main(argv):
    if len(argv) < 2 or len(argv) % 2:
        raise SystemExit(__doc__)
    json.dump(merge(list(zip(argv[0::2], argv[1::2]))), sys.stdout, indent=1)
    print()


if __name__ == "__main__":
    main(sys.argv[1:])
