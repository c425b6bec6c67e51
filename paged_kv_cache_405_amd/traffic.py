"""Measured HBM traffic of a decode call, from profiler counters.

A record holds, for one benchmark configuration (workload, resolved path,
layout), the bytes the decode call's kernels moved to and from HBM per call,
from two ``rocprofv3 --pmc`` runs of bench.py (FETCH_SIZE, then WRITE_SIZE,
in KiB per dispatch).  Each counter is scaled by what it reads for a plain
1 GiB device copy (``bench.py --copy-calibration``), since a counter need not
count bytes one to one.  The record carries a digest of the kernel sources
and build flags: once they change, the measurement no longer describes the
code and ``lookup`` returns None.

    python -m paged_kv_cache_405_amd.traffic record --workload llama7b \\
        --partition -1 --kernel 1 --layout bhtd [--shared-blocks] [--prefix-pass] \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
        --command "rocprofv3 ..." [--command ...]

DIR is a rocprofv3 output directory holding ``*counter_collection.csv``.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
DEFAULT_PATH = os.path.join(ROOT, "profiles", "hbm_traffic.json")
COPY_BYTES = 1 << 30


def sources_digest() -> str:
    """sha256 over the kernel sources and the build script (flags included)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*"))) + [os.path.join(PKG, "build.py")]
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _counter(dirname: str, counter: str) -> dict[str, float]:
    """Mean value per dispatch of one counter, per kernel name."""
    files = glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {dirname}")
    vals = defaultdict(list)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def _decode_kernels(per_kernel: dict[str, float]) -> dict[str, float]:
    """The kernels a decode call launches (the append kernel is not one)."""
    return {k: v for k, v in per_kernel.items() if "pa::" in k and "append" not in k}


def _copy_kib(dirname: str, counter: str) -> float:
    per = {k: v for k, v in _counter(dirname, counter).items() if "copy" in k.lower()}
    if not per:
        raise ValueError(f"no copy kernel in {dirname}")
    return max(per.values())


def _key(r):
    return (r["workload"], r["partition"], r["kernel"], r["layout"], r.get("shared_blocks", False),
            r.get("prefix_pass", False))


def record(path, workload, partition, kernel, layout, shared_blocks, fetch_dir, write_dir, copy_fetch_dir,
           copy_write_dir, commands, prefix_pass=False):
    fetch = _decode_kernels(_counter(fetch_dir, "FETCH_SIZE"))
    write = _decode_kernels(_counter(write_dir, "WRITE_SIZE"))
    fetch_scale = COPY_BYTES / 1024 / _copy_kib(copy_fetch_dir, "FETCH_SIZE")
    write_scale = COPY_BYTES / 1024 / _copy_kib(copy_write_dir, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        kernels[k] = {"FETCH_SIZE_kib": fetch.get(k, 0.0), "WRITE_SIZE_kib": write.get(k, 0.0)}
    read_bytes = sum(v["FETCH_SIZE_kib"] for v in kernels.values()) * 1024 * fetch_scale
    write_bytes = sum(v["WRITE_SIZE_kib"] for v in kernels.values()) * 1024 * write_scale
    entry = {
        "workload": workload, "partition": int(partition), "kernel": int(kernel), "layout": layout,
        "shared_blocks": bool(shared_blocks), "prefix_pass": bool(prefix_pass),
        "sources_sha256": sources_digest(),
        "fetch_scale": fetch_scale, "write_scale": write_scale,
        "kernels": kernels,
        "read_bytes_per_call": read_bytes, "write_bytes_per_call": write_bytes,
        "bytes_per_call": read_bytes + write_bytes,
        "commands": list(commands),
    }
    data = {"records": []}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    data["records"] = [r for r in data["records"] if _key(r) != _key(entry)] + [entry]
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return entry


def lookup(workload, partition, kernel, layout, shared_blocks=False, path=DEFAULT_PATH, prefix_pass=False):
    """The record for this configuration if it was measured on the current sources, else None."""
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    digest = sources_digest()
    for r in data.get("records", []):
        if _key(r) == (workload, partition, kernel, layout, bool(shared_blocks), bool(prefix_pass)):
            return r if r["sources_sha256"] == digest else None
    return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("record")
    r.add_argument("--path", default=DEFAULT_PATH)
    r.add_argument("--workload", required=True)
    r.add_argument("--partition", type=int, required=True)
    r.add_argument("--kernel", type=int, required=True)
    r.add_argument("--layout", default="bhtd")
    r.add_argument("--shared-blocks", action="store_true")
    r.add_argument("--prefix-pass", action="store_true", help="the call was pa_decode_shared_prefix")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--copy-fetch", required=True)
    r.add_argument("--copy-write", required=True)
    r.add_argument("--command", action="append", default=[])
    a = ap.parse_args()
    e = record(a.path, a.workload, a.partition, a.kernel, a.layout, a.shared_blocks, a.fetch, a.write,
               a.copy_fetch, a.copy_write, a.command, prefix_pass=a.prefix_pass)
    print(json.dumps({k: e[k] for k in ("workload", "partition", "kernel", "bytes_per_call", "read_bytes_per_call",
                                        "write_bytes_per_call", "fetch_scale", "write_scale")}))


if __name__ == "__main__":
    main()
