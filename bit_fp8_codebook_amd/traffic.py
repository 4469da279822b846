"""Turn rocprofv3 counter dumps into per-launch HBM traffic for bench.py.

    python -m bit_fp8_codebook_amd.traffic FETCH.csv WRITE.csv > profiles/traffic.json

FETCH.csv / WRITE.csv are the `*_counter_collection.csv` files of two
`rocprofv3 --pmc FETCH_SIZE` and `rocprofv3 --pmc WRITE_SIZE` runs of
`bench.py --calibrate-copy`.  Each counter is scaled by what it reads for the
plain 256 MiB device-to-device copy in the same run (known bytes read and
written), which corrects for the share of the memory system the counter
block observes.  The result is keyed by a hash of the library sources, so it
is ignored as soon as a kernel changes.
"""
from __future__ import annotations

import collections
import csv
import json
import sys

COPY_BYTES = 256 << 20


def per_kernel(path, counter):
    vals = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return vals


def short(name):
    for key in ("linear_kernel<", "wide_kernel<", "pack_kernel", "unpack_kernel", "budget_topk_kernel", "topk_kernel",
                "combine_kernel", "quantize_kernel", "shortlist_chunks", "rescore_kernel", "copyBuffer"):
        if key in name:
            i = name.index(key)
            return name[i:name.index(">", i) + 1] if key.endswith("<") and ">" in name[i:] else key
    return name[:60]


def main(fetch_csv, write_csv):
    sys.path.insert(0, __import__("os").path.dirname(__import__("os").path.dirname(__file__)))
    from bench import source_hash
    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    copy_f = [v for k, vs in f.items() if "copyBuffer" in k for v in vs]
    copy_w = [v for k, vs in w.items() if "copyBuffer" in k for v in vs]
    # the calibration copy is the largest copy in the run
    fs = COPY_BYTES / 1024 / max(copy_f)
    ws = COPY_BYTES / 1024 / max(copy_w)
    out = {"source_hash": source_hash(), "fetch_scale": fs, "write_scale": ws, "kernels": {}}
    for k in f:
        if "copyBuffer" in k:
            continue
        rd = sum(f[k]) / len(f[k]) * 1024 * fs
        wr = (sum(w[k]) / len(w[k]) * 1024 * ws) if k in w else None
        out["kernels"][short(k)] = {"read_bytes": round(rd), "write_bytes": round(wr) if wr else None,
                                    "dispatches": len(f[k])}
    json.dump(out, sys.stdout, indent=1)


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
