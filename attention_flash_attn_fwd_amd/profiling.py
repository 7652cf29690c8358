"""Helpers that turn rocprofv3 result databases into the short text and JSON
summaries kept under profiles/.  Nothing here runs attention; it only reads
rocprofv3's SQLite output, plus one plain copy kernel used to calibrate the
HBM byte counters.

    python -m attention_flash_attn_fwd_amd.profiling copy [--mib 1024] [--reps 5]
        run torch's elementwise copy of a MiB-sized float32 buffer REPS times
        (the calibration kernel: reads and writes exactly MiB MiB per launch)
    python -m attention_flash_attn_fwd_amd.profiling trace DB --cmd "..." --title "..." --out F
        per-kernel call count and mean/min/max duration from a --kernel-trace run
    python -m attention_flash_attn_fwd_amd.profiling traffic --fetch DB --write DB
        --copy-fetch DB --copy-write DB --copy-mib 1024 --cmd "..." --out-json F --out-txt F
        HBM bytes per launch from FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch),
        each scaled by the factor that maps the copy kernel's reading to its true size
"""
from __future__ import annotations

import argparse
import collections
import hashlib
import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_flash_attn_fwd_amd", "csrc")

# kernel-name fragment -> (record key, source file whose hash the record carries)
TRACKED = {
    "prefill_bf16_kernel<128, true, false, false>": ("prefill_bf16", "prefill_bf16.hip"),
    "decode_native_kernel<128>": ("decode_native", "decode_paged.hip"),
    "decode_split_kernel<128>": ("decode_split", "decode_paged.hip"),
    "decode_merge_kernel<128>": ("decode_merge", "decode_paged.hip"),
}


def source_hash(name: str) -> str:
    with open(os.path.join(CSRC, name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def short_name(name: str) -> str:
    s = name.replace("attn::(anonymous namespace)::", "").replace("void ", "")
    i = s.find("(")
    return s[:i] if i > 0 else s


def kernel_rows(db_path: str, by_grid: bool = False):
    cur = sqlite3.connect(db_path).cursor()
    if by_grid:
        q = """select name || ' [' || grid_x || 'x' || grid_y || 'x' || grid_z || ']', count(*),
                      avg(duration), min(duration), max(duration), sum(duration)
               from kernels group by name, grid_x, grid_y, grid_z order by sum(duration) desc"""
    else:
        q = """select name, count(*), avg(duration), min(duration), max(duration), sum(duration)
               from kernels group by name order by sum(duration) desc"""
    return list(cur.execute(q))


def counter_means(db_path: str, counter: str):
    """Mean over dispatches of a counter (summed over its instances), per kernel."""
    cur = sqlite3.connect(db_path).cursor()
    cols = [d[0] for d in cur.execute("select * from counters_collection limit 1").description]
    ci = {c: i for i, c in enumerate(cols)}
    name_col = ci.get("kernel_name", ci.get("name"))
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for r in cur.execute("select * from counters_collection"):
        if r[ci["counter_name"]] != counter:
            continue
        per[r[name_col]][r[ci["dispatch_id"]]] += float(r[ci["value"]])
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def find_db(path: str) -> str:
    if os.path.isfile(path):
        return path
    hits = []
    for d, _, files in os.walk(path):
        hits += [os.path.join(d, f) for f in files if f.endswith("_results.db")]
    if len(hits) != 1:
        raise SystemExit(f"expected one *_results.db under {path}, found {hits}")
    return hits[0]


def cmd_copy(a):
    import torch
    n = a.mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(a.reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"copy calibration: {a.reps} launches of torch.neg over {a.mib} MiB float32 "
          f"(reads {a.mib} MiB, writes {a.mib} MiB each)", flush=True)


def cmd_trace(a):
    rows = kernel_rows(find_db(a.db), a.by_grid)
    tot = sum(r[5] for r in rows) or 1
    w = 64 if a.by_grid else 48
    out = [a.title, "", "Command (repo root, TMPDIR=/tmp):", "  " + a.cmd, "",
           f"{'kernel' + (' [grid]' if a.by_grid else ''):<{w}} {'calls':>5} {'avg_us':>9} "
           f"{'min_us':>9} {'max_us':>9} {'pct':>6}"]
    for n, c, av, mn, mx, s in rows:
        name = short_name(n.split(' [')[0]) + (' [' + n.split(' [')[1] if ' [' in n else '')
        out.append(f"{name[:w]:<{w}} {c:>5} {av / 1e3:>9.2f} {mn / 1e3:>9.2f} "
                   f"{mx / 1e3:>9.2f} {100 * s / tot:>6.2f}")
    if a.note:
        out += ["", a.note]
    text = "\n".join(out) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


def _copy_factor(db, counter, mib):
    m = counter_means(find_db(db), counter)
    cands = [(k, v) for k, v in m.items() if "elementwise" in k or "neg" in k.lower()]
    if not cands:
        raise SystemExit(f"no copy kernel in {db}: {list(m)}")
    (k, (kib, n)) = max(cands, key=lambda kv: kv[1][0])
    return (mib * 1024.0) / kib, kib, n


def cmd_traffic(a):
    ff, fk, fn = _copy_factor(a.copy_fetch, "FETCH_SIZE", a.copy_mib)
    wf, wk, wn = _copy_factor(a.copy_write, "WRITE_SIZE", a.copy_mib)
    fetch = counter_means(find_db(a.fetch), "FETCH_SIZE")
    write = counter_means(find_db(a.write), "WRITE_SIZE")
    rec = {"_calibration": {
        "copy_kernel": f"torch.neg over {a.copy_mib} MiB float32",
        "FETCH_SIZE_KiB": round(fk, 1), "fetch_factor": round(ff, 5),
        "WRITE_SIZE_KiB": round(wk, 1), "write_factor": round(wf, 5), "dispatches": [fn, wn]},
        "_command": a.cmd}
    lines = ["HBM traffic per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (separate runs),",
             "each scaled by the ratio true/measured of a plain copy kernel of known size.", "",
             "Command (repo root, TMPDIR=/tmp):", "  " + a.cmd, "",
             f"calibration: copy of {a.copy_mib} MiB reads FETCH_SIZE {fk:.0f} KiB "
             f"(factor {ff:.4f}), WRITE_SIZE {wk:.0f} KiB (factor {wf:.4f})", "",
             f"{'kernel':<40} {'fetch_MB':>10} {'write_MB':>10} {'total_MB':>10} {'n':>4}"]
    for frag, (key, src) in TRACKED.items():
        fk_ = [k for k in fetch if frag in k]
        wk_ = [k for k in write if frag in k]
        if not fk_ or not wk_:
            continue
        fb = fetch[fk_[0]][0] * 1024 * ff
        wb = write[wk_[0]][0] * 1024 * wf
        rec[key] = {"kernel": frag, "source": src, "source_sha256_16": source_hash(src),
                    "fetch_bytes": round(fb), "write_bytes": round(wb),
                    "bytes_per_launch": round(fb + wb), "dispatches": fetch[fk_[0]][1]}
        lines.append(f"{frag:<40} {fb / 1e6:>10.2f} {wb / 1e6:>10.2f} {(fb + wb) / 1e6:>10.2f} "
                     f"{fetch[fk_[0]][1]:>4}")
    with open(a.out_json, "w") as f:
        json.dump(rec, f, indent=1)
    with open(a.out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sp = ap.add_subparsers(dest="cmd_name", required=True)
    c = sp.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=5)
    t = sp.add_parser("trace")
    t.add_argument("db")
    t.add_argument("--cmd", required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--note", default="")
    t.add_argument("--by-grid", action="store_true",
                   help="one row per (kernel, grid) instead of per kernel")
    t.add_argument("--out", required=True)
    r = sp.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        r.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    r.add_argument("--copy-mib", type=int, default=1024)
    r.add_argument("--cmd", required=True)
    r.add_argument("--out-json", required=True)
    r.add_argument("--out-txt", required=True)
    a = ap.parse_args()
    {"copy": cmd_copy, "trace": cmd_trace, "traffic": cmd_traffic}[a.cmd_name](a)


if __name__ == "__main__":
    main()
