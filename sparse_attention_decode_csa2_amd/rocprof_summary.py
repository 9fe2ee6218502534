"""Condense rocprofv3 CSV output into the short text summaries kept under
profiles/.

    python -m sparse_attention_decode_csa2_amd.rocprof_summary stats DIR --command "..."
        Kernel table (calls, average / min / max duration, share of GPU time)
        from the *_kernel_stats.csv of a `rocprofv3 --kernel-trace --stats` run.

    python -m sparse_attention_decode_csa2_amd.rocprof_summary traffic \
        --fetch DIR1 --write DIR2 --kernel REGEX --calib REGEX --calib-bytes N \
        --workload NAME --source attn.hip --command "..."
        HBM bytes per launch of the kernels matching REGEX, from two `--pmc`
        runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch).  With --kernel
        given more than once, the figure is the sum over the kernels of their
        averages per dispatch: the bytes of one call that launches each of
        them once (the attention kernel and its split combine).  Each counter is
        scaled by the factor that makes it read N bytes for a calibration
        kernel of known size (a plain device copy: N bytes read, N written).
        The output is what bench.py reads as roofline.traffic, tagged with a
        hash of the kernel's source so that a stale measurement is ignored.

    python -m sparse_attention_decode_csa2_amd.rocprof_summary counters DIR \
        --kernel REGEX --workload NAME --command "..."
        Average per dispatch of every counter of a `--pmc` run for the kernels
        matching REGEX (instances summed), and the matrix-core utilisation
        SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs) when both
        are present (ROCm's MfmaUtil): the rows hold GRBM_GUI_ACTIVE, the busy
        cycles of the kernel, summed over MI355X's 8 XCDs, and the MFMA busy
        cycles summed over its 256 x 4 SIMDs.
"""

import argparse
import csv
import glob
import hashlib
import os
import re
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def _local_sources(name):
    """The source file and every header of csrc/ it includes, directly or
    through another (in the order first met)."""
    seen, todo = [], [name]
    while todo:
        f = todo.pop(0)
        if f in seen:
            continue
        seen.append(f)
        with open(os.path.join(CSRC, f)) as fh:
            todo += re.findall(r'^#include "([^"]+)"', fh.read(), flags=re.M)
    return seen


def kernel_source_hash(name):
    """Hash of a kernel source file plus the local headers it includes (less
    csa2_internal.h, which only declares the host-side launch functions).
    `name` may join several files with '+' (a stage whose launches come from
    more than one file)."""
    h = hashlib.sha256()
    files = []
    for part in name.split("+"):
        files += [f for f in _local_sources(part) if f not in files]
    for f in files:
        if f == "csa2_internal.h":
            continue
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits


def _short(name, width=96):
    """Kernel name without its trailing parameter list, cut to `width`."""
    name = name.strip()
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i].rstrip()
                break
    return name if len(name) <= width else name[:width - 3] + "..."


def stats(args):
    rows = []
    for f in _find(args.dir, "kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# rocprofv3 kernel statistics", f"# command: {args.command}", "#",
           f"{'kernel':<98} {'calls':>7} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'share%':>7}"]
    for r in rows:
        out.append(f"{_short(r['Name']):<98} {int(r['Calls']):>7} {float(r['AverageNs']) / 1e3:>9.3f} "
                   f"{float(r['MinNs']) / 1e3:>9.3f} {float(r['MaxNs']) / 1e3:>9.3f} "
                   f"{float(r['Percentage']):>7.2f}")
    print("\n".join(out))


def _counter_means(d, counter):
    """Average counter value per dispatch (instances summed), keyed by kernel name."""
    acc = {}
    for f in _find(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")))
                acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    per = {}
    for (name, _), v in acc.items():
        per.setdefault(name, []).append(v)
    return per


def _pick(per, regex, what):
    hits = {k: v for k, v in per.items() if re.search(regex, k)}
    if not hits:
        raise SystemExit(f"no {what} kernel matches {regex!r}")
    vals = [x for v in hits.values() for x in v]
    return sum(vals) / len(vals), len(vals), sorted(hits)


def traffic(args):
    f_per = _counter_means(args.fetch, "FETCH_SIZE")
    w_per = _counter_means(args.write, "WRITE_SIZE")
    cf, _, cnames = _pick(f_per, args.calib, "calibration")
    cw, _, _ = _pick(w_per, args.calib, "calibration")
    f_scale = args.calib_bytes / (cf * 1024.0)
    w_scale = args.calib_bytes / (cw * 1024.0)
    kf = kw = 0.0
    nf, nw, knames = [], [], []
    for rx in args.kernel:
        f, n1, names = _pick(f_per, rx, "measured")
        w, n2, _ = _pick(w_per, rx, "measured")
        kf += f
        kw += w
        nf.append(str(n1))
        nw.append(str(n2))
        knames += names
    fetch = kf * 1024.0 * f_scale
    write = kw * 1024.0 * w_scale
    print("\n".join([
        f"# HBM traffic per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch),",
        f"# each scaled so that the calibration copy reads and writes exactly {args.calib_bytes} bytes",
        f"# command: {args.command}",
        f"workload: {args.workload}",
        f"kernel: {' | '.join(_short(k, 200) for k in knames)}",
        f"calibration_kernel: {' | '.join(_short(k, 200) for k in cnames)}",
        f"source_file: {args.source}",
        f"source_hash: {kernel_source_hash(args.source)}",
        f"dispatches: {'+'.join(nf)} fetch, {'+'.join(nw)} write",
        f"fetch_kib_raw: {kf:.1f}",
        f"write_kib_raw: {kw:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"fetch_bytes_per_launch: {fetch:.0f}",
        f"write_bytes_per_launch: {write:.0f}",
        f"bytes_per_launch: {fetch + write:.0f}",
    ]))


def counters(args):
    names = set()
    for f in _find(args.dir, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                names.add(r["Counter_Name"])
    vals = {}
    knames = []
    for c in sorted(names):
        v, nd, kn = _pick(_counter_means(args.dir, c), args.kernel, "measured")
        vals[c] = (v, nd)
        knames = kn
    out = ["# rocprofv3 counters, average per dispatch",
           f"# command: {args.command}",
           f"workload: {args.workload}",
           f"kernel: {' | '.join(_short(k, 200) for k in knames)}"]
    for c, (v, nd) in vals.items():
        out.append(f"{c}: {v:.1f}  ({nd} dispatches)")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and "GRBM_GUI_ACTIVE" in vals:
        busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"][0]
        simd_cycles = vals["GRBM_GUI_ACTIVE"][0] / 8.0 * 1024.0
        out.append(f"mfma_util: {busy / simd_cycles:.4f}  (matrix-core busy cycles over the kernel's SIMD cycles)")
    print("\n".join(out))


def read_traffic(path):
    """Parse a traffic summary written by `traffic` into a dict of strings."""
    rec = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, action="append")
    t.add_argument("--calib", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    {"stats": stats, "traffic": traffic, "counters": counters}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
