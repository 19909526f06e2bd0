"""Summarise rocprofv3 output of bench.py into short text plus HBM traffic.

    python -m kv_cache_quantization_05_amd.rocpd_summary --workload W \
        --trace DIR [--fetch DIR --write DIR] --out-txt FILE [--traffic-json FILE] \
        [--command "..."]

--trace: a `rocprofv3 --kernel-trace --stats` run; --fetch / --write: runs of
`rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE` over `bench.py
--calibrate-copy`.  The calibrating dispatch is the largest runtime buffer
copy (copyBuffer) of the run, which moves exactly 1 GiB; each counter is scaled by
1 GiB / (its reading for that dispatch), so the reported bytes are in the
units of a plain copy of known size.  Databases are deleted after reading
(they are large); the text keeps the figures used.

Launch groups: one tq_attend_decode call runs the split-K kernel, the merge
kernel and (for QJL keys or the generic path) the query kernel, so its
figures are sums over those kernels per merge dispatch; one
tq_attend_prefill call runs the query kernel, the prefill kernel and the
rotation back, counted per prefill dispatch; one tq_encode call
runs one encode kernel, so its figures are averages over encode dispatches
(K and V launches alike); one tq_scores call runs the query kernel, the
scorer and (top-k) the list merge, counted per scorer dispatch.  The query
kernel belongs to tq_scores in runs without decode kernels.
"""

import argparse
import glob
import hashlib
import json
import os
import re
import sqlite3

PKG = os.path.dirname(os.path.abspath(__file__))
GIB = 1 << 30

GROUPS = {
    "attend_decode": re.compile(r"attend_mfma_kernel|attend_partial_kernel|attend_merge_kernel|query_prep_kernel"),
    "attend_prefill": re.compile(r"prefill(32)?_kernel|rotate_back_kernel"),
    "encode": re.compile(r"encode_kernel|encode_qjl_kernel|encode_qjl_mfma_kernel|encode_mfma_kernel|encode_var_kernel|encode_haar_kernel"),
    "scores": re.compile(r"scores_tile32_kernel|scores_mfma_kernel|scores_topk_kernel|scores_full_kernel|topk_merge_kernel"),
}
# dispatches that count launches of each group
ANCHORS = {"attend_decode": re.compile(r"attend_merge_kernel"), "encode": GROUPS["encode"],
           "attend_prefill": re.compile(r"prefill(32)?_kernel"),
           "scores": re.compile(r"scores_tile32_kernel|scores_mfma_kernel|scores_topk_kernel|scores_full_kernel")}
QUERY = re.compile(r"query_prep_kernel")
DECODE_ONLY = re.compile(r"attend_mfma_kernel|attend_partial_kernel|attend_merge_kernel")
PREFILL = re.compile(r"prefill(32)?_kernel")
_has_decode = [True]
_has_prefill = [False]


# HIP sources whose kernels make up each launch group; every header and host
# source counts for every group.  Recorded traffic is valid only for the
# hash of its group's sources.
GROUP_SOURCES = {
    "attend_decode": ("tq_attend.hip", "tq_attend_dims.hip", "tq_attend_mfma.hip"),
    "attend_prefill": ("tq_prefill.hip", "tq_attend.hip", "tq_attend_dims.hip"),
    "encode": ("tq_encode.hip", "tq_encode_qjl.hip", "tq_encode_var.hip"),
    "scores": ("tq_scores.hip", "tq_scores32.hip", "tq_attend.hip", "tq_attend_dims.hip"),
}


def kernel_source_hash(group=None):
    """Hash of the sources a launch group's kernels are built from (every
    source when group is None)."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    own = GROUP_SOURCES.get(group)
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".h", ".cpp")) or (f.endswith(".hip") and (own is None or f in own)):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def short(name):
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    name = re.sub(r"\(.*", "", name)
    return name.replace("void ", "")[-90:]


def _dbs(d):
    return sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True))


def read_trace(d):
    """Per kernel name: name, calls, avg, min, max (us), vgpr, lds, scratch,
    blocks, median (us)."""
    rows = []
    for db in _dbs(d):
        con = sqlite3.connect(db)
        for r in con.execute(
                "select name, count(*), avg(duration)/1000.0, min(duration)/1000.0, max(duration)/1000.0, "
                "max(vgpr_count), max(lds_size), max(scratch_size), "
                "max(grid_x*grid_y*grid_z/(workgroup_x*workgroup_y*workgroup_z)) "
                "from kernels group by name order by sum(duration) desc"):
            ds = sorted(x[0] / 1000.0 for x in con.execute("select duration from kernels where name = ?", (r[0],)))
            rows.append(tuple(r) + (ds[len(ds) // 2],))
        con.close()
    return rows


def read_counter(d, counter):
    """[(kernel, n, avg, max)] per kernel name, plus per-dispatch values of the
    copy kernels (for calibration)."""
    per, copies = [], []
    for db in _dbs(d):
        con = sqlite3.connect(db)
        per += list(con.execute(
            "select kernel_name, count(*), avg(value), max(value) from counters_collection "
            "where counter_name = ? group by kernel_name", (counter,)))
        copies += [r[0] for r in con.execute(
            "select value from counters_collection where counter_name = ? and "
            "kernel_name like '%copyBuffer%'", (counter,))]
        con.close()
    return per, copies


def group_of(name):
    # the query kernel belongs to the call that ran it: decode, prefill or scores
    if QUERY.search(name) and not _has_decode[0]:
        return "attend_prefill" if _has_prefill[0] else "scores"
    for g, rx in GROUPS.items():
        if rx.search(name):
            return g
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--out-txt", required=True)
    ap.add_argument("--traffic-json")
    ap.add_argument("--command", default="")
    ap.add_argument("--keep-db", action="store_true")
    args = ap.parse_args()

    out = [f"# rocprofv3 summary: workload {args.workload}",
           "# kernel sources: " + ", ".join(f"{g} {kernel_source_hash(g)}" for g in GROUP_SOURCES)]
    if args.command:
        out.append(f"# commands: {args.command}")
    trace = read_trace(args.trace)
    _has_decode[0] = any(DECODE_ONLY.search(r[0]) for r in trace)
    _has_prefill[0] = any(PREFILL.search(r[0]) for r in trace)
    out.append("## kernel trace (durations in us)")
    out.append("kernel | calls | avg_us | min_us | max_us | vgpr | lds | scratch | blocks | median_us")
    per_group = {}
    for r in trace:
        out.append(f"{short(r[0])} | {r[1]} | {r[2]:.2f} | {r[3]:.2f} | {r[4]:.2f} | {r[5]} | {r[6]} | {r[7]} | {r[8]} | {r[9]:.2f}")
        g = group_of(r[0])
        if g:
            per_group.setdefault(g, []).append((r[0], r[1], r[2], r[9]))
    out.append("## per launch: total duration of the group's dispatches / launches (warm-up launches included);"
               " median: the sum over the group's kernels of (median duration x dispatches / launches)")
    launches = {}
    for g, ks in per_group.items():
        launches[g] = sum(k[1] for k in ks if ANCHORS[g].search(k[0]))
        n = max(launches[g], 1)
        total = sum(k[1] * k[2] for k in ks)
        med = sum(k[1] * k[3] for k in ks)
        out.append(f"{g}: {total / n:.2f} us per launch (median {med / n:.2f} us) over {launches[g]} launches "
                   f"({', '.join(f'{short(k[0])} x{k[1]}' for k in ks)})")

    traffic = {}
    for counter, d in (("FETCH_SIZE", args.fetch), ("WRITE_SIZE", args.write)):
        if not d:
            continue
        per, copies = read_counter(d, counter)
        if not copies or max(copies) <= 0:
            out.append(f"## {counter}: no copy dispatch to calibrate against")
            continue
        cal = (GIB / 1024.0) / max(copies)  # KiB of a 1 GiB copy / counter reading
        out.append(f"## {counter} (KiB per dispatch as read; calibration: the 1 GiB copy reads "
                   f"{max(copies):.0f}, factor {cal:.4f})")
        n_launch = {}
        for k, n, avg, mx in sorted(per, key=lambda r: -r[2] * r[1]):
            g = group_of(k)
            if g is None and "copy" not in k.lower():
                continue
            out.append(f"{short(k)} | n={n} | avg={avg:.1f} | max={mx:.1f} | calibrated bytes/dispatch={avg * cal * 1024:.4g}")
            if g:
                traffic.setdefault(g, {}).setdefault(counter, 0.0)
                traffic[g][counter] += n * avg * cal * 1024
                if ANCHORS[g].search(k):
                    n_launch[g] = n_launch.get(g, 0) + n
        for g in traffic:
            if counter in traffic[g]:
                traffic[g][counter] /= max(n_launch.get(g, 1), 1)
    if traffic:
        out.append("## traffic per launch (calibrated bytes)")
        for g, t in traffic.items():
            out.append(f"{g}: fetch {t.get('FETCH_SIZE', 0):.4g} B, write {t.get('WRITE_SIZE', 0):.4g} B, "
                       f"total {t.get('FETCH_SIZE', 0) + t.get('WRITE_SIZE', 0):.4g} B")
    txt = "\n".join(out) + "\n"
    os.makedirs(os.path.dirname(os.path.abspath(args.out_txt)), exist_ok=True)
    with open(args.out_txt, "w") as f:
        f.write(txt)
    print(txt)
    if args.traffic_json and traffic:
        rec = {}
        if os.path.exists(args.traffic_json):
            rec = json.load(open(args.traffic_json))
        for g, t in traffic.items():
            if "FETCH_SIZE" in t and "WRITE_SIZE" in t:
                rec[f"{args.workload}:{g}"] = {
                    "bytes_per_launch": int(t["FETCH_SIZE"] + t["WRITE_SIZE"]),
                    "fetch_bytes": int(t["FETCH_SIZE"]), "write_bytes": int(t["WRITE_SIZE"]),
                    "source_hash": kernel_source_hash(g)}
        with open(args.traffic_json, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
    if not args.keep_db:
        for d in (args.trace, args.fetch, args.write):
            if d:
                for db in _dbs(d):
                    os.remove(db)


if __name__ == "__main__":
    main()
