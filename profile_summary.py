"""Summaries of rocprofv3 output for profiles/.

  python profile_summary.py stats <kernel_stats.csv> <title> <command>
      Markdown table of a `rocprofv3 --kernel-trace --stats` run.

  python profile_summary.py traffic <fetch_counter_collection.csv>
      <write_counter_collection.csv> <kernel-substring> <name> <workload> <sources>
      <out-dir> <command-fetch> <command-write>
      HBM bytes per dispatch of a kernel from FETCH_SIZE and WRITE_SIZE runs
      (KiB per dispatch), each scaled by what the same counter reads for the
      plain 1 GiB device copies (`__amd_rocclr_copyBuffer`) that
      `bench.py --calibrate-copy` runs first: the copy reads and writes
      exactly 1 GiB. <sources>: the kernel's files under csrc/, comma-separated.
      Writes <out-dir>/traffic_<name>_<workload>.json (read by bench.py while
      those files are unchanged) and a markdown summary.

  python profile_summary.py kernels <kernel_stats.csv> <fetch csv> <write csv>
      <mfma csv> <workload> <commands-file>
      Per library kernel: mean duration (kernel trace), HBM bytes read and
      written per dispatch (FETCH_SIZE / WRITE_SIZE, scaled as above), the
      achieved HBM rate against 8 TB/s, and the MFMA pipe busy fraction
      (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE per XCD x 1024 SIMDs).
      Markdown on stdout.
"""
import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY = "__amd_rocclr_copyBuffer"
GIB_KIB = 1 << 20


def _find(path: str, suffix: str) -> str:
    if os.path.isfile(path):
        return path
    hits = sorted(glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {path}")
    return hits[0]


def stats(path: str, title: str, command: str) -> str:
    rows = list(csv.DictReader(open(_find(path, "kernel_stats.csv"))))
    out = [f"# {title}", "", "Command (from the repository root):", "", "```", command, "```", "",
           "| kernel | calls | avg µs | min µs | max µs | % of GPU time |",
           "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("dsmoe::(anonymous namespace)::", "")
        if len(name) > 110:
            name = name[:110]
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.2f} |")
    return "\n".join(out) + "\n"


def _per_dispatch(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter (values of one
    dispatch summed over the rows rocprofv3 wrote for it)."""
    acc = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(_find(path, "counter_collection.csv"))):
        if r["Counter_Name"] != counter:
            continue
        key = int(r["Dispatch_Id"])
        acc[key] += float(r["Counter_Value"])
        names[key] = r["Kernel_Name"]
    per = collections.defaultdict(list)
    for key in sorted(acc):
        per[names[key]].append(acc[key])
    return per


def _select(per, sub: str):
    hits = [(k, v) for k, v in per.items() if sub in k]
    if len(hits) != 1:
        raise SystemExit(f"{len(hits)} kernels match {sub!r}: {[k[:80] for k, _ in hits]}")
    return hits[0]


def sources_sha256(source: str) -> str:
    """One SHA-256 over the kernel's source files (comma-separated names under
    csrc/, hashed in the order given), so that a change to any of them marks
    the counters as stale. bench.py computes the same digest."""
    h = hashlib.sha256()
    for name in source.split(","):
        h.update(open(os.path.join(ROOT, "sparse_mixture_experts_gate_amd", "csrc", name),
                      "rb").read())
    return h.hexdigest()


def traffic(fetch_csv, write_csv, sub, name, workload, source, out_dir, cmd_f, cmd_w):
    pf, pw = _per_dispatch(fetch_csv, "FETCH_SIZE"), _per_dispatch(write_csv, "WRITE_SIZE")
    # the calibration copies are the three largest copy dispatches of each run
    cf = sorted(pf[COPY])[-3:]
    cw = sorted(pw[COPY])[-3:]
    f_scale = GIB_KIB / (sum(cf) / len(cf))
    w_scale = GIB_KIB / (sum(cw) / len(cw))
    kname, fv = _select(pf, sub)
    _, wv = _select(pw, sub)
    rd = sum(fv) / len(fv) * f_scale * 1024
    wr = sum(wv) / len(wv) * w_scale * 1024
    rec = {"kernel": kname, "workload": workload, "source": source,
           "source_sha256": sources_sha256(source),
           "fetch_scale": f_scale, "write_scale": w_scale,
           "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
           "bytes_per_launch": rd + wr, "dispatches": len(fv)}
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"traffic_{name}_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    md = [f"# HBM traffic of `{kname[:100]}`, {workload}", "",
          "Commands (from the repository root), one counter per run, then this summary:", "",
          "```", cmd_f, cmd_w,
          f"python profile_summary.py traffic <fetch csv> <write csv> {sub} {name} {workload} "
          f"{source} profiles", "```", "",
          f"Calibration: `bench.py --calibrate-copy` first runs three plain 1 GiB device copies "
          f"(`{COPY}`). On them FETCH_SIZE reads {sum(cf) / len(cf):.0f} KiB and WRITE_SIZE "
          f"{sum(cw) / len(cw):.0f} KiB for 1048576 KiB moved each way: scale factors "
          f"FETCH x{f_scale:.4f}, WRITE x{w_scale:.4f}.", "",
          "| dispatch | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) |", "|---|---|---|"]
    for i, (a, b) in enumerate(zip(fv, wv)):
        md.append(f"| {i} | {a:.0f} | {b:.0f} |")
    md += ["", f"Per launch (scaled, mean): read {rd / 1e9:.3f} GB, written {wr / 1e9:.3f} GB, "
               f"total {(rd + wr) / 1e9:.3f} GB."]
    with open(os.path.join(out_dir, f"hbm_traffic_{name}_{workload}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(rec))


HBM_PEAK = 8e12
N_XCD, N_SIMD = 8, 1024


def _means(path: str, counter: str):
    return {k: sum(v) / len(v) for k, v in _per_dispatch(path, counter).items()}


def kernels(stats_csv, fetch_csv, write_csv, mfma_csv, workload, cmd_file) -> str:
    dur = {r["Name"]: float(r["AverageNs"]) * 1e-9
           for r in csv.DictReader(open(_find(stats_csv, "kernel_stats.csv")))}
    pf, pw = _per_dispatch(fetch_csv, "FETCH_SIZE"), _per_dispatch(write_csv, "WRITE_SIZE")
    f_scale = GIB_KIB / (sum(sorted(pf[COPY])[-3:]) / 3)
    w_scale = GIB_KIB / (sum(sorted(pw[COPY])[-3:]) / 3)
    busy, grbm = _means(mfma_csv, "SQ_VALU_MFMA_BUSY_CYCLES"), _means(mfma_csv, "GRBM_GUI_ACTIVE")
    out = [f"# Per-kernel counters: {workload}", "",
           "Commands (from the repository root), one counter group per run, then this summary:",
           "", "```", open(cmd_file).read().strip(), "```", "",
           f"HBM bytes are FETCH_SIZE x {f_scale:.4f} and WRITE_SIZE x {w_scale:.4f} "
           "(calibrated on plain 1 GiB copies), per dispatch; GB/s uses the kernel-trace mean "
           "duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 "
           "SIMDs).", "",
           "| kernel | mean µs | read GB | written GB | HBM GB/s | % of 8 TB/s | MFMA busy |",
           "|---|---|---|---|---|---|---|"]
    for name in sorted(dur, key=lambda n: -dur[n]):
        if "dsmoe" not in name or name not in pf:
            continue
        rd = sum(pf[name]) / len(pf[name]) * f_scale * 1024
        wr = sum(pw[name]) / len(pw[name]) * w_scale * 1024 if name in pw else 0.0
        gbs = (rd + wr) / dur[name] / 1e9
        mf = ""
        if name in busy and grbm.get(name):
            mf = f"{busy[name] / (grbm[name] / N_XCD * N_SIMD):.1%}"
        short = name.replace("dsmoe::(anonymous namespace)::", "")[:70]
        out.append(f"| `{short}` | {dur[name] * 1e6:.1f} | {rd / 1e9:.4f} | {wr / 1e9:.4f} | "
                   f"{gbs:.0f} | {gbs * 1e9 / HBM_PEAK:.1%} | {mf} |")
    return "\n".join(out) + "\n"


def main(argv) -> int:
    if len(argv) >= 4 and argv[0] == "stats":
        sys.stdout.write(stats(argv[1], argv[2], argv[3]))
        return 0
    if len(argv) == 10 and argv[0] == "traffic":
        traffic(*argv[1:])
        return 0
    if len(argv) == 7 and argv[0] == "kernels":
        sys.stdout.write(kernels(*argv[1:]))
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
