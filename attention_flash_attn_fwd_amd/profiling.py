"""Measurement helpers: the workload launcher profiled under rocprofv3, and
the code that turns rocprofv3's result databases into the short text and
JSON summaries kept under profiles/.

    python -m attention_flash_attn_fwd_amd.profiling launch WORKLOAD [--reps 5] [--warmup 3]
        run one named workload (seeded inputs, the library's entry points)
        REPS times after WARMUP launches; the command that rocprofv3 wraps
    python -m attention_flash_attn_fwd_amd.profiling copy [--mib 1024] [--reps 5]
        run torch's elementwise copy of a MiB-sized float32 buffer REPS times
        (the calibration kernel: reads and writes exactly MiB MiB per launch)
    python -m attention_flash_attn_fwd_amd.profiling trace DB --cmd "..." --title "..." --out F
        per-kernel call count and mean/min/max duration from a --kernel-trace run
    python -m attention_flash_attn_fwd_amd.profiling traffic --fetch DB --write DB
        --copy-fetch DB --copy-write DB --copy-mib 1024 --cmd "..." --out-json F --out-txt F
        HBM bytes per launch from FETCH_SIZE / WRITE_SIZE runs (KiB per dispatch),
        each scaled by the factor that maps the copy kernel's reading to its true size
    python -m attention_flash_attn_fwd_amd.profiling counters --dir D --copy-fetch DB
        --copy-write DB --out-json F --out-txt F
        per workload under D (subfolders WORKLOAD/{trace,fetch,write,mfma}), the
        kernel time, calibrated HBM bytes and the MFMA-busy fraction per launch
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


# ---------------------------------------------------------------- workloads

# name -> (kernel-name fragment of its dominant kernel, source file, what a
# launch computes: ("flops", n) or ("bytes", n) filled in by launch())
WORKLOADS = ["gqa_causal_s8192", "mha_causal_s2048", "blockskip_s32768",
             "blockskip_s32768_stress", "chunked_prefill_paged", "paged_decode_gqa",
             "paged_decode_gqa_mfma", "paged_decode_gqa_fp8", "paged_decode_shared_prefix",
             "paged_decode_blockskip", "paged_decode_blockskip_stress",
             "paged_decode_blockskip_stress_rowmajor"]
KERNEL_OF = {
    "gqa_causal_s8192": "prefill_bf16_kernel<128, true, false, false>",
    "mha_causal_s2048": "prefill_bf16_kernel<128, true, false, false>",
    "blockskip_s32768": "prefill_bf16_kernel<128, true, true, false>",
    "blockskip_s32768_stress": "prefill_bf16_kernel<128, true, true, false>",
    "chunked_prefill_paged": "prefill_bf16_kernel<128, true, false, true>",
    "paged_decode_gqa": "decode_split_kernel<128>",
    "paged_decode_gqa_mfma": "decode_native_kernel<128>",
    "paged_decode_gqa_fp8": "decode_fp8_kernel<128, 2>",
    "paged_decode_shared_prefix": "decode_native_kernel<128>",
    "paged_decode_blockskip": "decode_skip_kernel<128>",
    "paged_decode_blockskip_stress": "decode_skip_kernel<128>",
    "paged_decode_blockskip_stress_rowmajor": "decode_skip_rm_kernel<128>",
}
SOURCE_OF = {k: ("decode_paged.hip" if k.startswith("paged") else "prefill_bf16.hip")
             for k in WORKLOADS}


def workload_runner(name: str):
    """(run, work) for a named workload: run() launches it once on the
    current stream; work = {"flops": F} (prefill, algorithmic) or
    {"kv_bytes": B} (decode, K/V bytes that must be read)."""
    import torch
    import attention_flash_attn_fwd_amd as A
    from workloads import (CONFIGS, blockskip_inputs, decode_inputs, fp8_decode_inputs,
                           paged_prefill_inputs, prefill_flops, prefill_inputs,
                           shared_prefix_decode_inputs)
    dev = "cuda"
    if name in ("gqa_causal_s8192", "mha_causal_s2048"):
        c = CONFIGS[name]
        w = prefill_inputs(c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], seed=c["seed"])
        q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((c["B"], c["Hq"], c["S"]), dtype=torch.float32, device=dev)
        return (lambda: A.attn_prefill(q, k, v, o, lse, True, w.scale),
                {"flops": prefill_flops(c["B"], c["Hq"], c["S"], c["D"], True)})
    if name.startswith("blockskip_s32768"):
        c = CONFIGS["blockskip_s32768"]
        stress = name.endswith("stress")
        w = blockskip_inputs(c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], seed=c["seed"],
                             amplitude=12.0 if stress else c["amplitude"],
                             boosted="second_half" if stress else c["boosted"])
        q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((c["B"], c["Hq"], c["S"]), dtype=torch.float32, device=dev)

        def run():
            A.attn_prefill_blockskip(q, k, v, o, lse, w.scale, c["lam"], 64, None, None)
            if not stress:  # the dense kernel on the same inputs, for comparison
                A.attn_prefill(q, k, v, o, lse, True, w.scale)
        return run, {"flops": prefill_flops(c["B"], c["Hq"], c["S"], c["D"], True)}
    if name == "chunked_prefill_paged":
        ctx_l, q_l = [3584] * 8, [512] * 8
        wc = paged_prefill_inputs(ctx_l, q_l, 32, 8, 128, seed=2005)
        cq, ccu = wc.q.to(dev), wc.cu_seqlens_q.to(dev)
        ckp, cvp = wc.k_pool.to(dev), wc.v_pool.to(dev)
        cbt, csk = wc.block_table.to(dev), wc.seq_lens_k.to(dev)
        co = torch.empty_like(cq)
        clse = torch.empty((int(wc.cu_seqlens_q[-1]), 32), dtype=torch.float32, device=dev)
        pairs = sum(qn * cx + qn * (qn + 1) // 2 for cx, qn in zip(ctx_l, q_l))
        return (lambda: A.attn_prefill_paged(cq, ccu, ckp, cvp, cbt, csk, co, clse,
                                             wc.max_seqlen_q, wc.scale),
                {"flops": 4 * 32 * 128 * pairs})
    c = CONFIGS["paged_decode_gqa"]
    if name == "paged_decode_shared_prefix":
        # 16 prompts of 1536 tokens, 4 samples each with U[1, 2048] own tokens
        ds = shared_prefix_decode_inputs(16, 4, c["Hq"], c["Hkv"], c["D"], seed=2004,
                                         prefix_len=1536, suffix_min=1, suffix_max=2048,
                                         layout="mfma")[0]
        sq, sbt, ssl = ds.q.to(dev), ds.block_table.to(dev), ds.seq_lens.to(dev)
        spools = [(ds.k_pool.to(dev), ds.v_pool.to(dev)) for _ in range(2)]
        sws = torch.empty(A.attn_decode_workspace_bytes(ds.N, c["Hq"], c["D"], ds.max_blocks,
                                                        16), dtype=torch.uint8, device=dev)
        so = torch.empty_like(sq)
        slse = torch.empty((ds.N, c["Hq"]), dtype=torch.float32, device=dev)
        sctr = [0]

        def run_shared():
            kp, vp = spools[sctr[0] % 2]
            sctr[0] += 1
            A.attn_decode_paged(sq, kp, vp, sbt, ssl, 16, so, slse, ds.scale, sws, layout="mfma")
        return run_shared, {"kv_bytes": ds.kv_bytes()}
    layout = "rowmajor" if name in ("paged_decode_gqa", "paged_decode_gqa_fp8",
                                    "paged_decode_blockskip_stress_rowmajor") else "mfma"
    skip = name.startswith("paged_decode_blockskip")
    amp = 12.0 if "stress" in name else 0.0
    d = decode_inputs(c["N"], c["Hq"], c["Hkv"], c["D"], seed=c["seed"], lmin=c["lmin"],
                      lmax=c["lmax"], layout=layout, sink_amplitude=amp,
                      sink_frac=1 / 64 if amp else 0.0)
    q, bt, sl = d.q.to(dev), d.block_table.to(dev), d.seq_lens.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((c["N"], c["Hq"]), dtype=torch.float32, device=dev)
    ws = torch.empty(A.attn_decode_workspace_bytes(c["N"], c["Hq"], c["D"], d.max_blocks, 16),
                     dtype=torch.uint8, device=dev)
    if name == "paged_decode_gqa_fp8":
        f8 = fp8_decode_inputs(c["N"], c["Hq"], c["Hkv"], c["D"], seed=c["seed"],
                               lmin=c["lmin"], lmax=c["lmax"])
        pools = [(f8.k_pool.to(dev), f8.v_pool.to(dev)) for _ in range(2)]
        ctr = [0]

        def run_fp8():
            kp, vp = pools[ctr[0] % 2]
            ctr[0] += 1
            A.attn_decode_paged_fp8(q, kp, vp, bt, sl, 16, o, lse, d.scale, f8.k_scale,
                                    f8.v_scale, ws)
        return run_fp8, {"kv_bytes": f8.kv_bytes()}
    # two copies of the pool, used alternately, so that the 256 MB last-level
    # cache cannot serve a launch's K/V from the previous one
    pools = [(d.k_pool.to(dev), d.v_pool.to(dev)) for _ in range(2)]
    ctr = [0]

    def run_dec():
        kp, vp = pools[ctr[0] % 2]
        ctr[0] += 1
        if skip:
            A.attn_decode_paged_blockskip(q, kp, vp, bt, sl, 16, o, lse, d.scale, 1e-3, ws,
                                          None, None, layout=layout)
        else:
            A.attn_decode_paged(q, kp, vp, bt, sl, 16, o, lse, d.scale, ws, layout=layout)
    return run_dec, {"kv_bytes": d.kv_bytes()}


def cmd_launch(a):
    import torch
    torch.cuda.set_device(0)
    run, work = workload_runner(a.workload)
    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    for _ in range(a.reps):
        run()
    torch.cuda.synchronize()
    print(f"launched {a.workload}: {a.warmup} warm-up + {a.reps} timed launches; {work}",
          flush=True)


N_XCC = 8          # MI355X: 8 XCDs; GRBM_GUI_ACTIVE is counted on each
N_SIMD = 1024      # 256 compute units x 4 SIMDs


def _per_dispatch(db_path: str, counter: str, frag: str, last: int):
    """(value, duration ns) of a counter for the last `last` dispatches of the
    kernels whose name contains frag (rocprofv3 sums a counter over its
    instances in counters_collection)."""
    cur = sqlite3.connect(db_path).cursor()
    rows = [(r[0], float(r[1]), float(r[2])) for r in cur.execute(
        "select dispatch_id, value, duration from counters_collection "
        "where counter_name = ? and kernel_name like ?", (counter, f"%{frag}%"))]
    rows.sort()
    return [(v, d) for _, v, d in rows[-last:]]


def _last_durations(db_path: str, frag: str, last: int):
    cur = sqlite3.connect(db_path).cursor()
    rows = list(cur.execute("select start, duration from kernels where name like ? order by start",
                            (f"%{frag}%",)))
    return [float(d) for _, d in rows[-last:]]


def cmd_counters(a):
    ff, fk, _ = _copy_factor(a.copy_fetch, "FETCH_SIZE", a.copy_mib)
    wf, wk, _ = _copy_factor(a.copy_write, "WRITE_SIZE", a.copy_mib)
    rec = {"_calibration": {"copy_kernel": f"torch.neg over {a.copy_mib} MiB float32",
                            "FETCH_SIZE_KiB": round(fk, 1), "fetch_factor": round(ff, 5),
                            "WRITE_SIZE_KiB": round(wk, 1), "write_factor": round(wf, 5)},
           "_commands": a.cmd_note, "_dispatches": f"the last {a.last} launches of each run"}
    lines = ["Counters per launch of each workload's dominant kernel (rocprofv3, MI355X), over",
             f"the last {a.last} launches of each run (earlier ones warm the chip up).", "",
             "Commands (repo root, TMPDIR=/tmp), for each WORKLOAD:", "  " + a.cmd_note, "",
             f"HBM bytes = FETCH_SIZE and WRITE_SIZE (KiB) x the factor that maps a "
             f"{a.copy_mib} MiB copy's reading to its true size (fetch {ff:.4f}, write {wf:.4f}).",
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs): the "
             "share of SIMD cycles the matrix cores worked,",
             "at the clock the chip ran (GRBM_GUI_ACTIVE per XCD / kernel time of the same "
             "dispatch); MFMA TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / kernel time.", "",
             f"{'workload':<38} {'trace us':>9} {'fetch MB':>9} {'write MB':>9} "
             f"{'MFMA busy':>9} {'clock GHz':>9} {'MFMA TF/s':>9}"]
    for wl in WORKLOADS:
        d = os.path.join(a.dir, wl)
        if not os.path.isdir(d):
            continue
        frag = KERNEL_OF[wl]
        r = {"kernel": frag, "source": SOURCE_OF[wl],
             "source_sha256_16": source_hash(SOURCE_OF[wl])}
        durs = _last_durations(find_db(os.path.join(d, "trace")), frag, a.last)
        us = sum(durs) / len(durs) / 1e3 if durs else None
        r["kernel_us"] = round(us, 2) if us else None
        if os.path.isdir(os.path.join(d, "fetch")):
            v = _per_dispatch(find_db(os.path.join(d, "fetch")), "FETCH_SIZE", frag, a.last)
            r["fetch_bytes"] = round(sum(x for x, _ in v) / len(v) * 1024 * ff) if v else None
        if os.path.isdir(os.path.join(d, "write")):
            v = _per_dispatch(find_db(os.path.join(d, "write")), "WRITE_SIZE", frag, a.last)
            r["write_bytes"] = round(sum(x for x, _ in v) / len(v) * 1024 * wf) if v else None
        if r.get("fetch_bytes") is not None and r.get("write_bytes") is not None:
            r["bytes_per_launch"] = r["fetch_bytes"] + r["write_bytes"]
        if os.path.isdir(os.path.join(d, "mfma")):
            db = find_db(os.path.join(d, "mfma"))
            b = _per_dispatch(db, "SQ_VALU_MFMA_BUSY_CYCLES", frag, a.last)
            g = _per_dispatch(db, "GRBM_GUI_ACTIVE", frag, a.last)
            m = _per_dispatch(db, "SQ_INSTS_VALU_MFMA_MOPS_BF16", frag, a.last)
            if b and g:
                busy = [x for x, _ in b]
                gui = [x / N_XCC for x, _ in g]
                r["mfma_busy_frac"] = round(sum(bb / (gg * N_SIMD) for bb, gg in zip(busy, gui)) /
                                            len(gui), 4)
                r["gui_active_cycles_per_xcd"] = round(sum(gui) / len(gui))
                r["clock_ghz"] = round(sum(gg / dd for gg, (_, dd) in zip(gui, g)) / len(g), 3)
                r["counter_run_kernel_us"] = round(sum(dd for _, dd in g) / len(g) / 1e3, 2)
            if m:
                r["mfma_flops_per_launch"] = round(sum(x for x, _ in m) / len(m) * 512)
                r["mfma_tflops"] = round(sum(x * 512 / (dd * 1e-9) for x, dd in m) / len(m) / 1e12,
                                         1)
        rec[wl] = r

        def f(x, k=1.0, nd=1):
            return f"{x / k:>9.{nd}f}" if isinstance(x, (int, float)) else f"{'-':>9}"
        lines.append(f"{wl:<38} {f(us, 1, 1)} {f(r.get('fetch_bytes'), 1e6)} "
                     f"{f(r.get('write_bytes'), 1e6)} {f(r.get('mfma_busy_frac'), 0.01)}% "
                     f"{f(r.get('clock_ghz'), 1, 3)} {f(r.get('mfma_tflops'), 1, 1)}")
    with open(a.out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    with open(a.out_txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cmd_pmc(a):
    """Counters per launch (mean over the last launches) of one kernel for
    several runs: one run directory per label."""
    labels = a.labels.split(",")
    dirs = a.dirs.split(",")
    counters = a.counters.split(",")
    assert len(labels) == len(dirs)
    lines = [a.title, "", "Command (repo root, TMPDIR=/tmp), for each run:", "  " + a.cmd, "",
             f"Mean per launch over the last {a.last} launches of the kernels named "
             f"*{a.kernel}*.", "",
             f"{'run':<28}" + "".join(f"{c:>22}" for c in counters)]
    for lab, d in zip(labels, dirs):
        db = find_db(d)
        vals = []
        for c in counters:
            v = _per_dispatch(db, c, a.kernel, a.last)
            vals.append(sum(x for x, _ in v) / len(v) if v else float("nan"))
        lines.append(f"{lab:<28}" + "".join(f"{x:>22.0f}" for x in vals))
    if a.note:
        lines += ["", a.note]
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    print(text, end="")


def main():
    ap = argparse.ArgumentParser()
    sp = ap.add_subparsers(dest="cmd_name", required=True)
    la = sp.add_parser("launch")
    la.add_argument("workload", choices=WORKLOADS)
    la.add_argument("--reps", type=int, default=5)
    la.add_argument("--warmup", type=int, default=3)
    co = sp.add_parser("counters")
    co.add_argument("--dir", required=True)
    co.add_argument("--copy-fetch", required=True)
    co.add_argument("--copy-write", required=True)
    co.add_argument("--copy-mib", type=int, default=1024)
    co.add_argument("--cmd-note", required=True)
    co.add_argument("--last", type=int, default=3, help="launches averaged, the last of each run")
    co.add_argument("--out-json", required=True)
    co.add_argument("--out-txt", required=True)
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
    pm = sp.add_parser("pmc")
    pm.add_argument("--dirs", required=True, help="comma-separated rocprofv3 output directories")
    pm.add_argument("--labels", required=True)
    pm.add_argument("--counters", required=True)
    pm.add_argument("--kernel", required=True, help="substring of the kernel name")
    pm.add_argument("--last", type=int, default=2)
    pm.add_argument("--title", required=True)
    pm.add_argument("--cmd", required=True)
    pm.add_argument("--note", default="")
    pm.add_argument("--out", required=True)
    r = sp.add_parser("traffic")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        r.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    r.add_argument("--copy-mib", type=int, default=1024)
    r.add_argument("--cmd", required=True)
    r.add_argument("--out-json", required=True)
    r.add_argument("--out-txt", required=True)
    a = ap.parse_args()
    {"copy": cmd_copy, "trace": cmd_trace, "traffic": cmd_traffic, "launch": cmd_launch,
     "counters": cmd_counters, "pmc": cmd_pmc}[a.cmd_name](a)


if __name__ == "__main__":
    main()
