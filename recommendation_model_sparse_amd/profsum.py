"""Summaries of rocprofv3 CSV output for the library's kernels.

    python -m recommendation_model_sparse_amd.profsum stats   DIR
    python -m recommendation_model_sparse_amd.profsum traffic WORKLOAD FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR [REV]
    python -m recommendation_model_sparse_amd.profsum counters DIR [COUNTER ...]

``stats`` prints the per-kernel table of a ``--kernel-trace --stats`` run.  ``traffic`` turns two
``--pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` runs into HBM bytes per launch, each counter scaled by
what it reads for a plain device copy of known size (``bench.py --copy-probe``: 1 GiB read and
1 GiB written), and ends with the machine-readable ``traffic-json:`` line that bench.py reads; the
line records the SHA-256 of each kernel's sources, so a later change to a kernel voids its bytes.
With REV (a git revision), the sources are hashed as they were at that revision: the one the
profiled tree was taken from.  ``counters`` prints per-kernel sums of any other counters (rocprofv3's derived ones included).
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = "recommendation_model_sparse_amd/csrc"
COMMON = [f"{CSRC}/common.h", "recommendation_model_sparse_amd/build.py"]

# source files each kernel family is built from (the traffic record is void once any changes)
KERNEL_SOURCES = {
    "pool": [f"{CSRC}/emb_bag_fwd.hip", f"{CSRC}/pool.h"],
    "emb_interact": [f"{CSRC}/emb_interact_fwd.hip", f"{CSRC}/pool.h", f"{CSRC}/gram.h"],
    "interact": [f"{CSRC}/interact.hip", f"{CSRC}/gram.h"],
    "bwd": [f"{CSRC}/emb_bag_bwd.hip"],
    "mlp": [f"{CSRC}/mlp.hip"],
    "fill": [f"{CSRC}/synth_fill.hip"],
    "probe": [f"{CSRC}/probe.hip"],
}


def family(short: str) -> str:
    if short.startswith("pool_"):
        return "pool"
    if short.startswith("emb_interact"):
        return "emb_interact"
    if short.startswith("interact"):
        return "interact"
    if short.startswith(("expand", "radix", "seg_", "zero_u32", "empty_outputs", "check_")):
        return "bwd"
    if short.startswith("fill"):
        return "fill"
    if short.startswith("probe"):
        return "probe"
    return "mlp"


def short_name(kernel: str) -> str:
    """'void dlrm::(anonymous namespace)::k_pool_wave_per_bag<1, 16, ...>(...)' -> 'pool_wave_per_bag'."""
    m = re.search(r"\bk_([A-Za-z0-9_]+)", kernel)
    return m.group(1) if m else kernel.split("(")[0].strip()


def template_name(kernel: str) -> str:
    m = re.search(r"\b(k_[A-Za-z0-9_]+(?:<[^()]*>)?)", kernel)
    return m.group(1) if m else kernel.split("(")[0].strip()


def sources_sha(files, rev=None) -> str:
    import subprocess
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(b"\0")
        if rev:
            h.update(subprocess.run(["git", "show", f"{rev}:{f}"], cwd=ROOT, check=True, capture_output=True).stdout)
        else:
            with open(os.path.join(ROOT, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def _csvs(d: str, suffix: str):
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def read_counters(d: str):
    """{(kernel, dispatch id): {counter: value}} from every counter_collection.csv under d."""
    out = collections.defaultdict(dict)
    for path in _csvs(d, "counter_collection.csv"):
        with open(path, newline="") as fh:
            for row in csv.DictReader(fh):
                key = (row["Kernel_Name"], row.get("Dispatch_Id") or row.get("Correlation_Id"))
                name = row["Counter_Name"]
                out[key][name] = out[key].get(name, 0.0) + float(row["Counter_Value"])
    return out


def per_kernel(d: str, counter: str):
    """{kernel: (dispatches, summed counter)}."""
    acc = collections.defaultdict(lambda: [0, 0.0])
    for (k, _), vals in read_counters(d).items():
        if counter in vals:
            acc[k][0] += 1
            acc[k][1] += vals[counter]
    return {k: (n, v) for k, (n, v) in acc.items()}


def copy_factor(d: str, counter: str, nbytes: int = 1 << 30) -> float:
    """Bytes per counter unit, from the plain copy of nbytes (read and written once)."""
    rec = per_kernel(d, counter)
    cands = [(n, v) for k, (n, v) in rec.items() if "copyBuffer" in k]
    if not cands:
        raise SystemExit(f"no copy kernel in {d}")
    n, v = max(cands, key=lambda x: x[1] / max(1, x[0]))
    return nbytes / (v / n)


def cmd_stats(d: str):
    rows = []
    for path in _csvs(d, "kernel_stats.csv"):
        with open(path, newline="") as fh:
            rows += list(csv.DictReader(fh))
    total = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("| kernel | calls | average (us) | min (us) | max (us) | share |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print(f"| `{template_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
              f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
              f"{100 * float(r['TotalDurationNs']) / total:.1f}% |")


def cmd_traffic(workload: str, fetch_dir: str, write_dir: str, cf_dir: str, cw_dir: str, rev=None):
    ff = copy_factor(cf_dir, "FETCH_SIZE")
    fw = copy_factor(cw_dir, "WRITE_SIZE")
    fr, wr = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    print(f"Calibration: FETCH_SIZE x{ff / 1024:.3f} KiB and WRITE_SIZE x{fw / 1024:.3f} KiB per unit "
          f"(a plain 1 GiB device copy reads 1 GiB and writes 1 GiB).\n")
    print("| kernel | dispatches | HBM read (MB/launch) | HBM write (MB/launch) |")
    print("|---|---|---|---|")
    fam = collections.defaultdict(lambda: [0, 0.0, 0.0])
    for k in sorted(set(fr) | set(wr), key=lambda k: -(fr.get(k, (1, 0))[1] / max(1, fr.get(k, (1, 0))[0]))):
        n = max(fr.get(k, (0, 0))[0], wr.get(k, (0, 0))[0])
        rb = fr[k][1] * ff / fr[k][0] if k in fr and fr[k][0] else 0.0
        wb = wr[k][1] * fw / wr[k][0] if k in wr and wr[k][0] else 0.0
        print(f"| `{template_name(k)}` | {n} | {rb / 1e6:.1f} | {wb / 1e6:.1f} |")
        if "k_" in k:
            s = short_name(k)
            e = fam[s]
            e[0] += n
            e[1] += rb * n
            e[2] += wb * n
    kernels = {}
    for s, (n, rb, wb) in sorted(fam.items()):
        files = KERNEL_SOURCES[family(s)] + COMMON
        kernels[s] = {"dispatches": n, "read_bytes": int(rb / n), "write_bytes": int(wb / n),
                      "sources": files, "source_sha256": sources_sha(files, rev)}
    print("\nPer-launch bytes by kernel (all instantiations together), with the SHA-256 of the sources the\n"
          "kernel is built from at the time of the run:\n")
    print("```")
    print("traffic-json: " + json.dumps({"workload": workload, "kernels": kernels}))
    print("```")


def cmd_counters(d: str, names):
    rec = read_counters(d)
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    cnt = collections.Counter()
    for (k, _), vals in rec.items():
        cnt[k] += 1
        for n, v in vals.items():
            acc[k][n] += v
    names = names or sorted({n for v in acc.values() for n in v})
    print("| kernel | dispatches | " + " | ".join(f"{n} (per launch)" for n in names) + " |")
    print("|---|---|" + "---|" * len(names))
    for k in sorted(acc, key=lambda k: template_name(k)):
        vals = " | ".join(f"{acc[k][n] / cnt[k]:.4g}" if n in acc[k] else "-" for n in names)
        print(f"| `{template_name(k)}` | {cnt[k]} | {vals} |")


def main(argv):
    if len(argv) >= 2 and argv[0] == "stats":
        cmd_stats(argv[1])
    elif len(argv) in (6, 7) and argv[0] == "traffic":
        cmd_traffic(*argv[1:])
    elif len(argv) >= 2 and argv[0] == "counters":
        cmd_counters(argv[1], argv[2:])
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
