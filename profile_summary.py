"""Summaries of rocprofv3 output for profiles/.

  python profile_summary.py stats <kernel_stats.csv> <title> <command>
      Markdown table of a `rocprofv3 --kernel-trace --stats` run.

  python profile_summary.py traffic <fetch dir> <write dir> <request dir>
      <kernel-substring> <load path> <name> <workload> <sources> <out-dir>
      <commands-file>
      HBM bytes per dispatch of a kernel: FETCH_SIZE (KiB per dispatch) scaled
      by what the same counter reads for the calibration read of the kernel's
      load path (<load path>: a key of bench.LOAD_CALIBRATION), WRITE_SIZE by
      what it reads for plain 1 GiB device copies; `bench.py --calibrate-loads
      --calibrate-copy` runs both first in every counter run. The <request
      dir> run counts L2-to-fabric read requests by size (TCC_EA0_RDREQ_sum,
      _32B_sum, _64B_sum, _128B_sum), a cross-check that needs no factor.
      <sources>: the kernel's files under csrc/, comma-separated. Writes
      <out-dir>/traffic_<name>_<workload>.json (read by bench.py while those
      files are unchanged) and a markdown summary.

  python profile_summary.py kernels <trace dir> <fetch dir> <write dir>
      <request dir> <mfma dir> <workload> <commands-file>
      Per library kernel: mean duration (kernel trace), bytes read per
      dispatch by request size and by plain FETCH_SIZE, bytes written
      (WRITE_SIZE scaled as above), the achieved HBM rate against 8 TB/s, and
      the MFMA pipe busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over
      GRBM_GUI_ACTIVE per XCD x 1024 SIMDs), after the calibration table.
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


# calibration reads of `bench.py --calibrate-loads` (bytes per launch) and the
# load path each stands for
sys.path.insert(0, ROOT)
from bench import LOAD_CALIBRATION  # noqa: E402

PATHS = {"hbm_dma_kernel<false>": "LDS-DMA, default policy",
         "hbm_dma_kernel<true>": "LDS-DMA, non-temporal",
         "hbm_read_kernel<false>": "register loads, default policy",
         "hbm_read_kernel<true>": "register loads, non-temporal"}
REQ = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
       "TCC_EA0_RDREQ_128B_sum")


def _cal_means(per, sub):
    """Mean per launch of the calibration kernel matching `sub`."""
    hits = [v for k, v in per.items() if sub in k]
    if len(hits) != 1:
        raise SystemExit(f"{len(hits)} calibration kernels match {sub!r}")
    return sum(hits[0]) / len(hits[0])


def _sized_bytes(req_csv):
    """{kernel: [bytes per dispatch]} from the read requests by size:
    32 R32 + 64 R64 + 128 R128, and {kernel: [requests not in any size
    class per dispatch]} (RDREQ - R32 - R64 - R128)."""
    per = {c: _per_dispatch(req_csv, c) for c in REQ}
    out, rest = {}, {}
    for k, tot in per[REQ[0]].items():
        r32, r64, r128 = per[REQ[1]][k], per[REQ[2]][k], per[REQ[3]][k]
        out[k] = [32 * a + 64 * b + 128 * c for a, b, c in zip(r32, r64, r128)]
        rest[k] = [t - a - b - c for t, a, b, c in zip(tot, r32, r64, r128)]
    return out, rest


def calibration(fetch_csv, write_csv, req_csv):
    """Scale factors and residuals of the calibration reads and copies:
    returns ({path kernel: FETCH_SIZE factor}, write factor, markdown lines)."""
    pf, pw = _per_dispatch(fetch_csv, "FETCH_SIZE"), _per_dispatch(write_csv, "WRITE_SIZE")
    sized, rest = _sized_bytes(req_csv)
    md = ["| calibration read (bytes per launch) | load path | FETCH_SIZE x 1024 / bytes | "
          "FETCH_SIZE factor | (32 R32 + 64 R64 + 128 R128) / bytes | unsized requests |",
          "|---|---|---|---|---|---|"]
    factors = {}
    for sub, nbytes in LOAD_CALIBRATION.items():
        fk = _cal_means(pf, sub) * 1024
        sb = _cal_means(sized, sub)
        factors[sub] = nbytes / fk
        md.append(f"| `{sub}` ({nbytes}) | {PATHS[sub]} | {fk / nbytes:.4f} | "
                  f"x{nbytes / fk:.4f} | {sb / nbytes:.4f} | {_cal_means(rest, sub):.0f} |")
    cf = sorted(pf[COPY])[-3:]
    cw = sorted(pw[COPY])[-3:]
    factors["copy"] = GIB_KIB / (sum(cf) / len(cf))
    w_scale = GIB_KIB / (sum(cw) / len(cw))
    md.append(f"| `{COPY}` (1 GiB each way) | copy | {1 / factors['copy']:.4f} | "
              f"x{factors['copy']:.4f} | | |")
    md += ["", f"WRITE_SIZE on the 1 GiB copies reads {sum(cw) / len(cw):.0f} KiB for 1048576 KiB "
               f"written: factor x{w_scale:.4f}."]
    return factors, w_scale, md


def sources_sha256(source: str) -> str:
    """One SHA-256 over the kernel's source files (comma-separated names under
    csrc/, hashed in the order given), so that a change to any of them marks
    the counters as stale. bench.py computes the same digest."""
    h = hashlib.sha256()
    for name in source.split(","):
        h.update(open(os.path.join(ROOT, "sparse_mixture_experts_gate_amd", "csrc", name),
                      "rb").read())
    return h.hexdigest()


def traffic(fetch_csv, write_csv, req_csv, sub, path, name, workload, source, out_dir, cmd_file):
    """HBM bytes per launch of the kernel matching `sub`: FETCH_SIZE scaled by
    the calibration read of its load path `path` (a LOAD_CALIBRATION key),
    WRITE_SIZE by the copies' factor; the request-size count beside it."""
    factors, w_scale, cal_md = calibration(fetch_csv, write_csv, req_csv)
    pf, pw = _per_dispatch(fetch_csv, "FETCH_SIZE"), _per_dispatch(write_csv, "WRITE_SIZE")
    sized, _ = _sized_bytes(req_csv)
    kname, fv = _select(pf, sub)
    _, wv = _select(pw, sub)
    _, sv = _select(sized, sub)
    f_scale = factors[path]
    rd = sum(fv) / len(fv) * f_scale * 1024
    wr = sum(wv) / len(wv) * w_scale * 1024
    rs = sum(sv) / len(sv)
    rec = {"kernel": kname, "workload": workload, "source": source,
           "source_sha256": sources_sha256(source), "load_path": path,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "read_bytes_per_launch": rd, "write_bytes_per_launch": wr,
           "read_bytes_by_request_size": rs,
           "bytes_per_launch": rd + wr, "dispatches": len(fv)}
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"traffic_{name}_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
    md = [f"# HBM traffic of `{kname[:100]}`, {workload}", "",
          "Commands (from the repository root), one counter group per run, then this summary:",
          "", "```", open(cmd_file).read().strip(), "```", "",
          "Calibration: every counter run first reads known byte counts through each load "
          "path of the library (`bench.py --calibrate-loads`) and makes three plain 1 GiB "
          "device copies. FETCH_SIZE of this kernel is scaled by the factor of its own load "
          f"path ({PATHS.get(path, path)}); the request-size count (32, 64 and 128-byte "
          "read requests from L2 to the fabric, times their sizes) needs no factor and is "
          "given beside it.", ""] + cal_md + [
          "", "| dispatch | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | read by request size (GB) |",
          "|---|---|---|---|"]
    for i, (a, b, c) in enumerate(zip(fv, wv, sv)):
        md.append(f"| {i} | {a:.0f} | {b:.0f} | {c / 1e9:.3f} |")
    md += ["", f"Per launch (mean): read {rd / 1e9:.3f} GB (FETCH_SIZE x{f_scale:.4f}), "
               f"{rs / 1e9:.3f} GB by request size; written {wr / 1e9:.3f} GB; total "
               f"{(rd + wr) / 1e9:.3f} GB."]
    with open(os.path.join(out_dir, f"hbm_traffic_{name}_{workload}.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(rec))


HBM_PEAK = 8e12
N_XCD, N_SIMD = 8, 1024


def _means(path: str, counter: str):
    return {k: sum(v) / len(v) for k, v in _per_dispatch(path, counter).items()}


def kernels(stats_csv, fetch_csv, write_csv, req_csv, mfma_csv, workload, cmd_file) -> str:
    dur = {r["Name"]: float(r["AverageNs"]) * 1e-9
           for r in csv.DictReader(open(_find(stats_csv, "kernel_stats.csv")))}
    factors, w_scale, cal_md = calibration(fetch_csv, write_csv, req_csv)
    pw = _per_dispatch(write_csv, "WRITE_SIZE")
    pf = _per_dispatch(fetch_csv, "FETCH_SIZE")
    sized, _ = _sized_bytes(req_csv)
    busy, grbm = _means(mfma_csv, "SQ_VALU_MFMA_BUSY_CYCLES"), _means(mfma_csv, "GRBM_GUI_ACTIVE")
    out = [f"# Per-kernel counters: {workload}", "",
           "Commands (from the repository root), one counter group per run, then this summary:",
           "", "```", open(cmd_file).read().strip(), "```", "",
           "Read bytes per dispatch come from the L2-to-fabric read requests by size "
           "(32 R32 + 64 R64 + 128 R128); the calibration reads below, one per load path, "
           "show how close that count comes to the bytes a kernel of known traffic reads, and "
           "what plain FETCH_SIZE would need as a factor on each path. Written bytes are "
           f"WRITE_SIZE x {w_scale:.4f} (calibrated on plain 1 GiB copies). GB/s uses the "
           "kernel-trace mean duration; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
           "(GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs).", ""] + cal_md + [
           "", "| kernel | mean µs | read GB | FETCH_SIZE GB (x1) | written GB | HBM GB/s | "
               "% of 8 TB/s | MFMA busy |",
           "|---|---|---|---|---|---|---|---|"]
    for name in sorted(dur, key=lambda n: -dur[n]):
        if "dsmoe" not in name or name not in sized:
            continue
        rd = sum(sized[name]) / len(sized[name])
        fk = sum(pf[name]) / len(pf[name]) * 1024 if name in pf else 0.0
        wr = sum(pw[name]) / len(pw[name]) * w_scale * 1024 if name in pw else 0.0
        gbs = (rd + wr) / dur[name] / 1e9
        mf = ""
        if name in busy and grbm.get(name):
            mf = f"{busy[name] / (grbm[name] / N_XCD * N_SIMD):.1%}"
        short = name.replace("dsmoe::(anonymous namespace)::", "")[:70]
        out.append(f"| `{short}` | {dur[name] * 1e6:.1f} | {rd / 1e9:.4f} | {fk / 1e9:.4f} | "
                   f"{wr / 1e9:.4f} | {gbs:.0f} | {gbs * 1e9 / HBM_PEAK:.1%} | {mf} |")
    return "\n".join(out) + "\n"


def main(argv) -> int:
    if len(argv) >= 4 and argv[0] == "stats":
        sys.stdout.write(stats(argv[1], argv[2], argv[3]))
        return 0
    if len(argv) == 11 and argv[0] == "traffic":
        traffic(*argv[1:])
        return 0
    if len(argv) == 8 and argv[0] == "kernels":
        sys.stdout.write(kernels(*argv[1:]))
        return 0
    print(__doc__, file=sys.stderr)
    return 2


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
