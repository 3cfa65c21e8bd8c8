"""Summaries of rocprofv3 runs of bench.py: per-kernel average durations
(``--kernel-trace --stats``) and HBM bytes per dispatch (``--pmc FETCH_SIZE``,
then ``--pmc WRITE_SIZE``, each in KiB per dispatch).  The byte counters are
scaled by what they read for a plain device-to-device copy of 1 GiB, which
bench.py runs first under ``--copy-calibration``.

    python -m manifold_constrained_residuals_amd.profiling summarize \\
        --stats DIR --fetch DIR --write DIR --bench-log FILE --out profiles/NAME

writes ``NAME_kernels.md`` (the table and the commands) and ``NAME_traffic.json``
(bytes per launch of each pass).  bench.py reads the JSON for its roofline
``traffic`` field and reports null once the kernel sources differ from the
digest recorded there.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.abspath(__file__))

# the kernels each entry point launches (bench.py's passes)
PASS_KERNELS = {
    # the single-read pass where the shape allows it (C = 256 G, G a multiple of 4 up to
    # 32), else the two-pass path; a pass sums the kernels that ran
    "mhc_fwd_pre": ["k_sr_prep", "k_fwd_sr", "k_sr_finish", "k_wsplit", "k_coeffs_part",
                    "k_finish_pre"],
    "mhc_post_res": ["k_post_res"],
    "mhc_post_res_bwd": ["k_post_res_bwd"],
    # n = 4: the read map's gradient and the Sinkhorn backward in one launch, the
    # remaining logit gradients, then the coefficient backward and its reductions
    "mhc_bwd_pre": ["k_pre_bwd_sk16", "k_dz16", "k_bwd_mfma_dma", "k_reduce_parts"],
    # the steady-state layer's fused call: the transform variant of the single-read pass
    # (the layer size takes it)
    "mhc_post_res_fwd_pre": ["k_sr_prep", "k_fwd_sr_xf", "k_sr_finish"],
}
COPY_BYTES = 1 << 30          # bench.py --copy-calibration: a 1 GiB device copy
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _code_only(text: str) -> str:
    """Source text without comments and blank space, so that comment edits keep the
    digest.  The sources hold no string literal with a comment marker in it."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest() -> str:
    """sha256 over the code of the HIP sources and the public header (any change to
    the code, not to its comments, resets it)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "csrc", "*.hip")) +
                   glob.glob(os.path.join(ROOT, "csrc", "*.hpp")))
    files.append(os.path.join(os.path.dirname(ROOT), "include", "mhc.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def base_name(kernel: str) -> str:
    """The kernel's name without namespace and template arguments; the single-read
    kernel's transform variant (second template argument true) is k_fwd_sr_xf."""
    m = re.search(r"mhc::(\w+)", kernel)
    if not m:
        return kernel
    if m.group(1) == "k_fwd_sr" and re.search(r"k_fwd_sr<\d+, true>", kernel):
        return "k_fwd_sr_xf"
    return m.group(1)


def _one(pattern, d):
    hits = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no {pattern} under {d}")
    return hits[0]


def read_stats(d):
    """kernel -> (calls, average ns) from a --kernel-trace --stats csv run"""
    out = {}
    for r in csv.DictReader(open(_one("*kernel_stats.csv", d))):
        out[base_name(r["Name"])] = (int(r["Calls"]), float(r["AverageNs"]))
    return out


def read_counter(d, counter):
    """kernel -> list of per-dispatch values (KiB) of one counter; plus the copy
    calibration dispatch's value"""
    per = collections.defaultdict(list)
    copy = 0.0
    for r in csv.DictReader(open(_one("*counter_collection.csv", d))):
        if r["Counter_Name"] != counter:
            continue
        v = float(r["Counter_Value"])
        if r["Kernel_Name"] == COPY_KERNEL:
            copy = max(copy, v)
        else:
            per[base_name(r["Kernel_Name"])].append(v)
    return per, copy


def summarize(stats_dir, fetch_dir, write_dir, bench_log, out, commands):
    stats = read_stats(stats_dir)
    fetch, fcopy = read_counter(fetch_dir, "FETCH_SIZE")
    write, wcopy = read_counter(write_dir, "WRITE_SIZE")
    ff = COPY_BYTES / (fcopy * 1024.0)
    wf = COPY_BYTES / (wcopy * 1024.0)
    bench = None
    for line in open(bench_log):
        line = line.strip()
        if line.startswith("{") and '"metric"' in line:
            bench = json.loads(line)
    assert bench is not None, f"no bench JSON line in {bench_log}"
    cfg = bench["config"]
    T, n, C = cfg["T"], cfg["n"], cfg["C"]
    s = 2 if cfg["storage"] == "bf16" else 4
    from bench import algo_bytes_per_token, fused_algo_bytes_per_token   # noqa: E402
    algo = {k: v * T for k, v in algo_bytes_per_token(n, C, s).items()}
    algo.update({k: v * T for k, v in fused_algo_bytes_per_token(n, C, s).items()})

    kern = {}
    for k, (calls, avg) in stats.items():
        # this library's kernels and the copy the counters are calibrated on (torch's own
        # kernels for the inputs and the copy-ceiling measurement are left out)
        if not (k.startswith("k_") or k == COPY_KERNEL):
            continue
        fb = sum(fetch.get(k, [0.0])) / max(1, len(fetch.get(k, []))) * 1024.0 * ff
        wb = sum(write.get(k, [0.0])) / max(1, len(write.get(k, []))) * 1024.0 * wf
        kern[k] = dict(calls=calls, avg_us=avg / 1e3, fetch_bytes=fb, write_bytes=wb,
                       raw_fetch_kib=(sum(fetch.get(k, [0.0])) / max(1, len(fetch.get(k, [])))),
                       raw_write_kib=(sum(write.get(k, [0.0])) / max(1, len(write.get(k, [])))))
    passes = {}
    for p, ks in PASS_KERNELS.items():
        if p not in bench["per_call_ms"]:
            continue                                # a pass this run does not time
        present = [k for k in ks if k in kern]
        passes[p] = dict(
            kernels=present,
            prof_avg_us=sum(kern[k]["avg_us"] for k in present),
            event_avg_us=bench["per_call_ms"][p] * 1e3,
            fetch_bytes=sum(kern[k]["fetch_bytes"] for k in present),
            write_bytes=sum(kern[k]["write_bytes"] for k in present),
            algorithmic_bytes=algo[p])
        passes[p]["hbm_bytes"] = passes[p]["fetch_bytes"] + passes[p]["write_bytes"]

    traffic = dict(workload=cfg["workload"], T=T, n=n, C=C, storage=cfg["storage"],
                   source_digest=source_digest(), fetch_factor=ff, write_factor=wf,
                   passes=passes, kernels=kern, commands=commands,
                   bench_ms_per_step=bench["ms_per_step"])
    with open(out + "_traffic.json", "w") as fh:
        json.dump(traffic, fh, indent=1, sort_keys=True)

    L = []
    L.append(f"# {cfg['workload']}: kernel times and HBM traffic (T={T}, n={n}, C={C}, "
             f"{cfg['storage']} storage)\n")
    L.append("One MI355X.  Commands, from the repository root:\n")
    L.append("```")
    L.extend(commands)
    L.append("```\n")
    L.append(f"Counter calibration: the 1 GiB copy read {fcopy:.0f} KiB on FETCH_SIZE and "
             f"{wcopy:.0f} KiB on WRITE_SIZE, so fetch bytes = FETCH_SIZE x 1024 x {ff:.3f} and "
             f"write bytes = WRITE_SIZE x 1024 x {wf:.3f}.\n")
    L.append("## Per kernel (averages per dispatch)\n")
    L.append("| kernel | calls | avg us | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB (scaled) | GB/s |")
    L.append("|---|---:|---:|---:|---:|---:|---:|")
    for k, v in sorted(kern.items(), key=lambda kv: -kv[1]["avg_us"]):
        mb = (v["fetch_bytes"] + v["write_bytes"]) / 1e6
        gbs = mb * 1e6 / (v["avg_us"] * 1e-6) / 1e9 if v["avg_us"] > 0 else 0.0
        L.append(f"| {k} | {v['calls']} | {v['avg_us']:.1f} | {v['raw_fetch_kib']:.0f} | "
                 f"{v['raw_write_kib']:.0f} | {mb:.1f} | {gbs:.0f} |")
    L.append("\n## Per pass (entry point)\n")
    L.append("| pass | kernels | profiler us | HIP-event us | algorithmic MB | HBM MB | "
             "HBM / algorithmic | algorithmic GB/s (events) |")
    L.append("|---|---|---:|---:|---:|---:|---:|---:|")
    for p, v in passes.items():
        L.append(f"| {p} | {', '.join(v['kernels'])} | {v['prof_avg_us']:.1f} | "
                 f"{v['event_avg_us']:.1f} | {v['algorithmic_bytes'] / 1e6:.1f} | "
                 f"{v['hbm_bytes'] / 1e6:.1f} | {v['hbm_bytes'] / v['algorithmic_bytes']:.3f} | "
                 f"{v['algorithmic_bytes'] / (v['event_avg_us'] * 1e-6) / 1e9:.0f} |")
    L.append(f"\nbench.py{' --steady-only' if cfg.get('step') else ''} (no profiler): "
             f"{bench['ms_per_step']:.4f} ms per step, "
             f"{bench['value'] / 1e6:.2f} M tokens/s, {100 * bench['hbm_frac_of_peak']:.1f} % of "
             "8 TB/s on algorithmic bytes.\n")
    with open(out + "_kernels.md", "w") as fh:
        fh.write("\n".join(L) + "\n")
    return traffic


def load_traffic(path):
    """The recorded traffic, or None when missing or recorded for other sources."""
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    return t if t.get("source_digest") == source_digest() else None


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--stats", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--bench-log", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--command", action="append", default=[],
                   help="a command that produced the inputs (repeat; recorded verbatim)")
    a = ap.parse_args()
    t = summarize(a.stats, a.fetch, a.write, a.bench_log, a.out, a.command)
    print(json.dumps({p: round(v["hbm_bytes"] / v["algorithmic_bytes"], 3)
                      for p, v in t["passes"].items()}))


if __name__ == "__main__":
    import sys
    sys.path.insert(0, os.path.dirname(ROOT))
    main()
