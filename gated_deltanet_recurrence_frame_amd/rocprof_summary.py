"""Summaries of rocprofv3 output for libgdn's kernels.

  python -m gated_deltanet_recurrence_frame_amd.rocprof_summary copy [--bytes N]
      a plain device copy of known size (torch copy_), the calibration
      target for the HBM byte counters;
  python -m gated_deltanet_recurrence_frame_amd.rocprof_summary trace DB_OR_DIR [--title T]
      per-kernel dispatch count and average / min / max duration from a
      `rocprofv3 --kernel-trace --stats` run (rocpd SQLite database);
  python -m gated_deltanet_recurrence_frame_amd.rocprof_summary traffic \
          --fetch CSV --write CSV --copy-fetch CSV --copy-write CSV \
          [--copy-bytes N] [--json OUT]
      HBM bytes per dispatch from `rocprofv3 --pmc FETCH_SIZE` and
      `--pmc WRITE_SIZE` runs (KiB per dispatch), each scaled by what the
      same counter reads for the plain copy of known size;
  python -m gated_deltanet_recurrence_frame_amd.rocprof_summary counters CSV [--xcds 8 --cus 256]
      shader-unit utilisation per kernel from one `rocprofv3 --pmc` run with
      SQ_VALU_MFMA_BUSY_CYCLES, SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT,
      SQ_WAVE_CYCLES, SQ_WAIT_INST_ANY, SQ_INSTS_MFMA, SQ_INSTS_LDS and
      GRBM_GUI_ACTIVE.  GRBM_GUI_ACTIVE reads the busy cycles summed over the
      XCDs, so one XCD's cycles are GRBM_GUI_ACTIVE / xcds; MFMA busy is the
      fraction of the SIMDs' cycles (cus x 4 per XCD cycle) with the MFMA unit
      busy, LDS busy the fraction of the CUs' cycles with the LDS active.

Nothing here is on the compute path.
"""

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sqlite3
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# kernel (short name) -> (name fragment in the trace, source files it is built from)
KERNELS = {
    "gram": ("gram_kernel<0, 7, 2, true, 2, false, false>", ["gdn_gram.hip", "gdn_device.h", "gdn_internal.h"]),
    "scan": ("scan_kernel<0, 7, 0>", ["gdn_scan.hip", "gdn_device.h", "gdn_internal.h"]),
    "output": ("output_kernel<0, 7, false, 2, false>", ["gdn_output.hip", "gdn_device.h", "gdn_internal.h"]),
    # backward (bf16, head pairs): X_t and dQ; the reverse scan; dK, dV, dbeta, W_t, dgamma
    "xdq": ("xdq_kernel<7, 2, false>", ["gdn_bwd_xdq.hip", "gdn_device.h", "gdn_internal.h"]),
    "scan_rev": ("scan_kernel<0, 7, 1>", ["gdn_scan.hip", "gdn_device.h", "gdn_internal.h"]),
    "bwd_kv": ("bwd_kv_kernel<0, 7, 2, false>", ["gdn_backward.hip", "gdn_device.h", "gdn_internal.h"]),
}


def source_sha(kernel):
    h = hashlib.sha256()
    for f in KERNELS[kernel][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _find(path, pattern):
    if os.path.isfile(path):
        return path
    hits = sorted(glob.glob(os.path.join(path, "**", pattern), recursive=True))
    if not hits:
        raise FileNotFoundError("no %s under %s" % (pattern, path))
    return hits[0]


def trace_table(db_or_dir):
    db = _find(db_or_dir, "*_results.db")
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, count(*), avg(end-start), min(end-start), max(end-start), sum(end-start) "
        "from kernels group by name order by sum(end-start) desc").fetchall()
    return [(r[0], r[1], r[2] / 1e3, r[3] / 1e3, r[4] / 1e3, r[5] / 1e3) for r in rows]


def counter_means(csv_path, counter):
    acc = collections.defaultdict(list)
    with open(_find(csv_path, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _copy_counter(csv_path, counter):
    vals = counter_means(csv_path, counter)
    # the copy is the only (or the largest) kernel in the calibration run
    return max(vals.values())


def traffic(fetch, write, copy_fetch, copy_write, copy_bytes):
    f_scale = copy_bytes / (_copy_counter(copy_fetch, "FETCH_SIZE") * 1024.0)
    w_scale = copy_bytes / (_copy_counter(copy_write, "WRITE_SIZE") * 1024.0)
    fm = counter_means(fetch, "FETCH_SIZE")
    wm = counter_means(write, "WRITE_SIZE")
    out = {"_scale": {"fetch": f_scale, "write": w_scale, "copy_bytes": copy_bytes}}
    for short, (frag, _) in KERNELS.items():
        fk = [k for k in fm if frag in k]
        wk = [k for k in wm if frag in k]
        if not fk or not wk:
            continue
        rb = fm[fk[0]] * 1024.0 * f_scale
        wb = wm[wk[0]] * 1024.0 * w_scale
        out[short] = {"kernel": fk[0], "read_bytes_per_launch": round(rb),
                      "write_bytes_per_launch": round(wb),
                      "bytes_per_launch": round(rb + wb), "source_sha": source_sha(short)}
    return out


def counters(csv_path, xcds, cus):
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(_find(csv_path, "*counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            for short, (frag, _) in KERNELS.items():
                if frag in r["Kernel_Name"]:
                    acc[short][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = {}
    for short, d in acc.items():
        m = {c: sum(v) / len(v) for c, v in d.items()}
        cyc = m["GRBM_GUI_ACTIVE"] / xcds          # one XCD's busy cycles
        out[short] = {
            "mfma_busy": m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * cus * 4),
            "lds_busy": m["SQ_LDS_IDX_ACTIVE"] / (cyc * cus),
            "lds_bank_conflict_share": m["SQ_LDS_BANK_CONFLICT"] / max(1.0, m["SQ_LDS_IDX_ACTIVE"]),
            "wave_wait_share": m["SQ_WAIT_INST_ANY"] / max(1.0, m["SQ_WAVE_CYCLES"]),
            "mfma_insts": m["SQ_INSTS_MFMA"], "lds_insts": m["SQ_INSTS_LDS"],
            "xcd_cycles": cyc,
        }
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--bytes", type=int, default=1 << 30)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--title", default="kernel trace")
    tr = sub.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        tr.add_argument("--" + k.replace("_", "-"), required=True)
    tr.add_argument("--copy-bytes", type=int, default=1 << 30)
    tr.add_argument("--json", default=None)
    cn = sub.add_parser("counters")
    cn.add_argument("csv")
    cn.add_argument("--xcds", type=int, default=8)
    cn.add_argument("--cus", type=int, default=256)
    a = ap.parse_args(argv)

    if a.cmd == "copy":
        import torch
        src = torch.empty(a.bytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print("copied %d bytes x3" % a.bytes)
    elif a.cmd == "trace":
        rows = trace_table(a.db)
        print("| kernel | dispatches | avg us | min us | max us |")
        print("|---|---|---|---|---|")
        for r in rows:
            print("| `%s` | %d | %.1f | %.1f | %.1f |" % (r[0], r[1], r[2], r[3], r[4]))
    elif a.cmd == "counters":
        print("| kernel | MFMA busy | LDS busy | LDS bank-conflict share | wave cycles waiting | "
              "MFMA insts | LDS insts |")
        print("|---|---|---|---|---|---|---|")
        for k, r in counters(a.csv, a.xcds, a.cus).items():
            print("| %s | %.1f%% | %.1f%% | %.0f%% | %.0f%% | %.3g | %.3g |" % (
                k, 100 * r["mfma_busy"], 100 * r["lds_busy"], 100 * r["lds_bank_conflict_share"],
                100 * r["wave_wait_share"], r["mfma_insts"], r["lds_insts"]))
    else:
        out = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes)
        text = json.dumps(out, indent=1, sort_keys=True)
        if a.json:
            with open(a.json, "w") as f:
                f.write(text + "\n")
        print(text)


if __name__ == "__main__":
    sys.exit(main())
