"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]

One step = one pass over the hot path's two entry points: the causal GQA
prefill of the long-context workload (B=1, Hq=32, Hkv=8, S=8192, D=128,
bf16; the largest dense prefill that the workloads name) and the paged GQA
decode (64 sequences, lengths U[512,4096], Hq=32, Hkv=8, D=128, 16-token
blocks, row-major [block, head, slot, dim] pools).  Inputs are seeded
synthetic tensors already resident in HBM.  W untimed warm-up steps, then
exactly K timed steps bracketed by device synchronisations: the K decodes
back to back, then the K prefills, with HIP events before, between and
after them on the stream the kernels run on, which gives each kernel's mean
launch duration without per-launch marker gaps.  Prints ONE JSON line.

`value` is the prefill throughput in TFLOP/s (algorithmic flops
4*B*Hq*D*S(S+1)/2 over the prefill kernel's mean event time).  The MHA
S=2048 prefill (the Llama-2-7B attention shape), the decode's K/V
bandwidth and the other paths are reported under "secondary".  The fp64 CPU
oracle is timed on a bounded sample of the same prefill workload as
"cpu_baseline".  Counter figures (HBM bytes, MFMA-busy fraction, clock)
come from profiles/counters.json and are reported only while the kernel
source they were taken on is unchanged.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
GPU_SPIN_CYCLES = 4_000_000  # about 2 ms of GPU time before a timed region


def kernel_hash(name: str) -> str:
    p = os.path.join(ROOT, "attention_flash_attn_fwd_amd", "csrc", name)
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counters(workload: str):
    """The committed rocprofv3 counter record of a workload (HBM bytes per
    launch, MFMA-busy fraction, clock), or None if it is missing or the
    kernel source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("source_sha256_16") != kernel_hash(rec["source"]):
        return None
    return rec


def traffic_of(workload: str):
    rec = counters(workload)
    return rec.get("bytes_per_launch") if rec else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the measurements other than the step's two kernels")
    ap.add_argument("--cpu-heads", type=int, default=32,
                    help="query heads of the prefill workload the CPU oracle runs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle sample until this much time has passed")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(no collectives, no sharding); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_flash_attn_fwd_amd as A
    from workloads import (CONFIGS, blockskip_inputs, decode_inputs, paged_prefill_inputs,
                           prefill_flops, prefill_inputs, shared_prefix_decode_inputs,
                           fp8_decode_inputs)

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    A.load()

    # ---------------------------------------------------------------- inputs
    cp = CONFIGS["gqa_causal_s8192"]
    wp = prefill_inputs(cp["B"], cp["Hq"], cp["Hkv"], cp["S"], cp["D"], seed=cp["seed"])
    # two copies of Q/K/V (2 x 96 MiB), used alternately, so that a launch
    # does not start with its inputs in the 256 MB last-level cache
    pre_in = [(wp.q.to(dev), wp.k.to(dev), wp.v.to(dev)) for _ in range(2)]
    o = torch.empty_like(pre_in[0][0])
    lse = torch.empty((cp["B"], cp["Hq"], cp["S"]), dtype=torch.float32, device=dev)
    p_flops = prefill_flops(cp["B"], cp["Hq"], cp["S"], cp["D"], True)

    cd = CONFIGS["paged_decode_gqa"]
    wd = decode_inputs(cd["N"], cd["Hq"], cd["Hkv"], cd["D"], seed=cd["seed"], lmin=cd["lmin"],
                       lmax=cd["lmax"], block_size=cd["block_size"])
    dq = wd.q.to(dev)
    # two copies of the pool (2 x 623 MB), used alternately, for the same reason
    pools = [(wd.k_pool.to(dev), wd.v_pool.to(dev)) for _ in range(2)]
    dbt, dsl = wd.block_table.to(dev), wd.seq_lens.to(dev)
    do = torch.empty_like(dq)
    dlse = torch.empty((cd["N"], cd["Hq"]), dtype=torch.float32, device=dev)
    ws = torch.empty(A.attn_decode_workspace_bytes(cd["N"], cd["Hq"], cd["D"], wd.max_blocks, 16),
                     dtype=torch.uint8, device=dev)
    kv_bytes = wd.kv_bytes()

    def run_prefill(i):
        q, k, v = pre_in[i % 2]
        A.attn_prefill(q, k, v, o, lse, True, wp.scale)

    def run_decode(i):
        kp, vp = pools[i % 2]
        A.attn_decode_paged(dq, kp, vp, dbt, dsl, 16, do, dlse, wd.scale, ws)

    # ------------------------------------------------------------ timed steps
    # K steps = K decodes and K prefills.  The decodes are issued back to
    # back, then the prefills, with one HIP event before, between and after,
    # all on the stream the kernels are launched on (torch's current stream,
    # passed through the C ABI).  A marker between every pair of launches
    # would add an idle gap of about 10 us in front of each kernel.  The
    # decodes go first: right after a burst of back-to-back prefills the
    # chip's power state slows the memory-bound decode by about 5%, which a
    # measurement of the decode kernel should not include.
    # The chip's clocks rise over roughly the first 10 ms of sustained load
    # (a prefill measured right after 1.5 ms of warm-up ran about 10% slower
    # than after 30 ms), so the default warm-up is 50 steps (about 30 ms).
    for i in range(args.warmup):
        run_prefill(i)
        run_decode(i)
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # a short GPU-side spin ahead of the first event lets the host queue the
    # launches before the timed region starts, so the first kernel does not
    # wait for the host
    torch.cuda._sleep(GPU_SPIN_CYCLES)
    e0.record()
    for i in range(args.steps):
        run_decode(i)
    e1.record()
    for i in range(args.steps):
        run_prefill(i)
    e2.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_s = e0.elapsed_time(e1) * 1e-3 / args.steps
    pre_s = e1.elapsed_time(e2) * 1e-3 / args.steps
    pre_tflops = p_flops / pre_s / 1e12
    dec_gbps = kv_bytes / dec_s / 1e9

    secondary = {
        "paged_decode_gqa": {
            "kv_GBps": round(dec_gbps, 1), "frac_hbm_peak": round(dec_gbps / PEAK_HBM_GBPS, 4),
            "us_per_launch": round(dec_s * 1e6, 2),
            "kv_bytes": kv_bytes, "launches": "decode_split + decode_merge",
            "pool_layout": "rowmajor", "traffic": traffic_of("paged_decode_gqa"),
        },
    }

    def time_it(fn, reps, warm=2):
        """Mean time per launch of `reps` back-to-back launches (HIP events).
        Short launches get more of both: at least about 30 ms of warm-up
        launches (the clock takes some ms of load to settle) and about 10 ms
        of timed ones."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        t1 = max(time.perf_counter() - t0, 1e-6)
        warm = max(warm, min(1000, math.ceil(0.03 / t1)))
        reps = max(reps, min(1000, math.ceil(0.01 / t1)))
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(GPU_SPIN_CYCLES)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    if not args.no_secondary:
        # the same cache in the MFMA-native pool layout (register-direct kernel)
        wr = decode_inputs(cd["N"], cd["Hq"], cd["Hkv"], cd["D"], seed=cd["seed"],
                           lmin=cd["lmin"], lmax=cd["lmax"], block_size=cd["block_size"],
                           layout="mfma")
        rpools = [(wr.k_pool.to(dev), wr.v_pool.to(dev)) for _ in range(2)]
        ctr = [0]

        def run_native():
            kp, vp = rpools[ctr[0] % 2]
            ctr[0] += 1
            A.attn_decode_paged(dq, kp, vp, dbt, dsl, 16, do, dlse, wd.scale, ws, layout="mfma")
        mr = time_it(run_native, 20)
        secondary["paged_decode_gqa_mfma_pools"] = {
            "kv_GBps": round(kv_bytes / mr / 1e9, 1),
            "frac_hbm_peak": round(kv_bytes / mr / 1e9 / PEAK_HBM_GBPS, 4),
            "us_per_launch": round(mr * 1e6, 2), "launches": "decode_native + decode_merge",
            "traffic": traffic_of("paged_decode_gqa_mfma")}
        del rpools

        # the same cache with FP8 (E4M3) pools, one fp32 scale per pool: half
        # the bytes per cached element (q, table and lengths are the same)
        f8 = fp8_decode_inputs(cd["N"], cd["Hq"], cd["Hkv"], cd["D"], seed=cd["seed"],
                               lmin=cd["lmin"], lmax=cd["lmax"])
        fpools = [(f8.k_pool.to(dev), f8.v_pool.to(dev)) for _ in range(2)]
        fctr = [0]

        def run_fp8():
            kp, vp = fpools[fctr[0] % 2]
            fctr[0] += 1
            A.attn_decode_paged_fp8(dq, kp, vp, dbt, dsl, 16, do, dlse, wd.scale, f8.k_scale,
                                    f8.v_scale, ws)
        mf = time_it(run_fp8, 20)
        fbytes = f8.kv_bytes()
        secondary["paged_decode_gqa_fp8_kv"] = {
            "kv_GBps": round(fbytes / mf / 1e9, 1),
            "frac_hbm_peak": round(fbytes / mf / 1e9 / PEAK_HBM_GBPS, 4),
            "us_per_launch": round(mf * 1e6, 2), "kv_bytes": fbytes,
            "speedup_vs_bf16_kv": round(dec_s / mf, 3), "traffic": traffic_of("paged_decode_gqa_fp8"),
            "note": "E4M3 codes, one fp32 scale per pool; same q, table and lengths"}
        del fpools

        # shared prompts (copy-on-write block tables): 16 prompts of 1536
        # tokens, 4 samples each with U[1, 2048] own tokens; the kernel reads
        # every sequence's logical K/V, shared blocks once per sequence
        ds, _ = shared_prefix_decode_inputs(16, 4, cd["Hq"], cd["Hkv"], cd["D"], seed=2004,
                                            prefix_len=1536, suffix_min=1, suffix_max=2048,
                                            layout="mfma")
        sq, sbt, ssl = ds.q.to(dev), ds.block_table.to(dev), ds.seq_lens.to(dev)
        spools = [(ds.k_pool.to(dev), ds.v_pool.to(dev)) for _ in range(2)]
        sws = torch.empty(A.attn_decode_workspace_bytes(ds.N, cd["Hq"], cd["D"], ds.max_blocks, 16),
                          dtype=torch.uint8, device=dev)
        so = torch.empty_like(sq)
        slse = torch.empty((ds.N, cd["Hq"]), dtype=torch.float32, device=dev)
        sctr = [0]

        def run_shared():
            kp, vp = spools[sctr[0] % 2]
            sctr[0] += 1
            A.attn_decode_paged(sq, kp, vp, sbt, ssl, 16, so, slse, ds.scale, sws, layout="mfma")
        ms = time_it(run_shared, 20)
        logical = ds.kv_bytes()
        unique = ds.num_blocks * cd["Hkv"] * 16 * cd["D"] * 2 * 2
        secondary["paged_decode_shared_prefix"] = {
            "logical_kv_GBps": round(logical / ms / 1e9, 1), "us_per_launch": round(ms * 1e6, 2),
            "logical_kv_bytes": logical, "unique_kv_bytes": unique,
            "traffic": traffic_of("paged_decode_shared_prefix"),
            "note": "16 prompts x 4 samples, 1536-token shared prompt, U[1,2048] own tokens"}
        del spools

        # block skip inside the decode: the decode workload itself, and a
        # labelled stress input with attention sinks (amplitude 12 on a seeded
        # dimension at token 0 and 1/64 of the cached tokens), lambda 1e-3
        for label, amp, lay in (("paged_decode_blockskip", 0.0, "mfma"),
                                ("paged_decode_blockskip_stress_sinks", 12.0, "mfma"),
                                ("paged_decode_blockskip_stress_sinks_rowmajor", 12.0, "rowmajor")):
            wb = decode_inputs(cd["N"], cd["Hq"], cd["Hkv"], cd["D"], seed=cd["seed"],
                               lmin=cd["lmin"], lmax=cd["lmax"], layout=lay,
                               sink_amplitude=amp, sink_frac=1 / 64 if amp else 0.0)
            bq, bbt, bsl = wb.q.to(dev), wb.block_table.to(dev), wb.seq_lens.to(dev)
            bpools = [(wb.k_pool.to(dev), wb.v_pool.to(dev)) for _ in range(2)]
            bcnt = torch.zeros(1, dtype=torch.int64, device=dev)
            bctr = [0]

            def run_dense():
                kp, vp = bpools[bctr[0] % 2]
                bctr[0] += 1
                A.attn_decode_paged(bq, kp, vp, bbt, bsl, 16, do, dlse, wb.scale, ws, layout=lay)

            def run_skip():
                kp, vp = bpools[bctr[0] % 2]
                bctr[0] += 1
                A.attn_decode_paged_blockskip(bq, kp, vp, bbt, bsl, 16, do, dlse, wb.scale, 1e-3,
                                              ws, None, None, layout=lay)
            md = time_it(run_dense, 20)
            mk = time_it(run_skip, 20)
            bcnt.zero_()
            A.attn_decode_paged_blockskip(bq, *bpools[0], bbt, bsl, 16, do, dlse, wb.scale, 1e-3,
                                          ws, None, bcnt, layout=lay)
            torch.cuda.synchronize()
            blocks = int(((wb.seq_lens.to(torch.int64) + 15) // 16).sum()) * cd["Hkv"]
            frac = int(bcnt.item()) / blocks
            kvb = wb.kv_bytes()
            secondary[label] = {
                "skipped_fraction": round(frac, 6), "skipped_blocks": int(bcnt.item()),
                "blocks": blocks, "lambda": 1e-3,
                "us_per_launch": round(mk * 1e6, 2), "dense_us_per_launch": round(md * 1e6, 2),
                "speedup_vs_dense": round(md / mk, 3),
                "logical_kv_GBps": round(kvb / mk / 1e9, 1),
                "read_kv_GBps": round(kvb * (1 - 0.5 * frac) / mk / 1e9, 1), "pool_layout": lay}
            secondary[label]["traffic"] = traffic_of(
                {"paged_decode_blockskip": "paged_decode_blockskip",
                 "paged_decode_blockskip_stress_sinks": "paged_decode_blockskip_stress",
                 "paged_decode_blockskip_stress_sinks_rowmajor":
                     "paged_decode_blockskip_stress_rowmajor"}[label])
            del bpools

        # chunked prefill over the paged cache: 8 sequences with 3584 cached
        # tokens and a new 512-token chunk each (GQA 32/8, D=128, row-major pools)
        ctx_l, q_l = [3584] * 8, [512] * 8
        wc = paged_prefill_inputs(ctx_l, q_l, cd["Hq"], cd["Hkv"], cd["D"], seed=2005)
        cq, ccu = wc.q.to(dev), wc.cu_seqlens_q.to(dev)
        ckp, cvp = wc.k_pool.to(dev), wc.v_pool.to(dev)
        cbt, csk = wc.block_table.to(dev), wc.seq_lens_k.to(dev)
        co = torch.empty_like(cq)
        clse = torch.empty((wc.total_q, cd["Hq"]), dtype=torch.float32, device=dev)
        mc = time_it(lambda: A.attn_prefill_paged(cq, ccu, ckp, cvp, cbt, csk, co, clse,
                                                  wc.max_seqlen_q, wc.scale), 10)
        pairs = sum(qn * c + qn * (qn + 1) // 2 for c, qn in zip(ctx_l, q_l))
        fc = 4 * cd["Hq"] * cd["D"] * pairs
        secondary["chunked_prefill_paged"] = {
            "TFLOPs": round(fc / mc / 1e12, 1), "frac_mfma_peak": round(fc / mc / 1e12 / PEAK_BF16_TFLOPS, 4),
            "us_per_launch": round(mc * 1e6, 1), "flops": fc,
            "counters": counters("chunked_prefill_paged"),
            "note": "8 seqs x (3584 cached + 512 new) tokens, Hq=32 Hkv=8 D=128, bottom-right causal"}
        del ckp, cvp

        # the MHA prefill at the Llama-2-7B attention shape (two rotating copies)
        c2 = CONFIGS["mha_causal_s2048"]
        w2 = prefill_inputs(c2["B"], c2["Hq"], c2["Hkv"], c2["S"], c2["D"], seed=c2["seed"])
        in2 = [(w2.q.to(dev), w2.k.to(dev), w2.v.to(dev)) for _ in range(2)]
        o2 = torch.empty_like(in2[0][0])
        l2 = torch.empty((c2["B"], c2["Hq"], c2["S"]), dtype=torch.float32, device=dev)
        c2ctr = [0]

        def run_c2():
            q2, k2, v2 = in2[c2ctr[0] % 2]
            c2ctr[0] += 1
            A.attn_prefill(q2, k2, v2, o2, l2, True, w2.scale)
        m2 = time_it(run_c2, 20)
        f2 = prefill_flops(c2["B"], c2["Hq"], c2["S"], c2["D"], True)
        secondary["mha_causal_s2048"] = {
            "TFLOPs": round(f2 / m2 / 1e12, 1), "frac_mfma_peak": round(f2 / m2 / 1e12 / PEAK_BF16_TFLOPS, 4),
            "us_per_launch": round(m2 * 1e6, 1), "counters": counters("mha_causal_s2048"),
            "note": "B=4 Hq=Hkv=32 S=2048 D=128 causal (Llama-2-7B attention shape)"}
        del in2, o2, l2

        c5 = CONFIGS["blockskip_s32768"]
        for label, amp, boosted in (("blockskip_s32768", c5["amplitude"], c5["boosted"]),
                                    ("blockskip_s32768_stress_amp12_second_half", 12.0,
                                     "second_half")):
            w5 = blockskip_inputs(1, c5["Hq"], c5["Hkv"], c5["S"], c5["D"], seed=c5["seed"],
                                  amplitude=amp, boosted=boosted)
            q5, k5, v5 = w5.q.to(dev), w5.k.to(dev), w5.v.to(dev)
            o5 = torch.empty_like(q5)
            l5 = torch.empty((1, c5["Hq"], c5["S"]), dtype=torch.float32, device=dev)
            cnt = torch.zeros(1, dtype=torch.int64, device=dev)
            m5 = time_it(lambda: A.attn_prefill_blockskip(q5, k5, v5, o5, l5, w5.scale,
                                                             c5["lam"], 64, None, cnt), 3, warm=1)
            cnt.zero_()
            A.attn_prefill_blockskip(q5, k5, v5, o5, l5, w5.scale, c5["lam"], 64, None, cnt)
            md = time_it(lambda: A.attn_prefill(q5, k5, v5, o5, l5, True, w5.scale), 3, warm=1)
            torch.cuda.synchronize()
            nT = c5["S"] // 64
            live = c5["Hq"] * nT * (nT + 1) // 2
            skipped = int(cnt.item())
            f5 = prefill_flops(1, c5["Hq"], c5["S"], c5["D"], True)
            # executed flops: Q.K^T on every live tile, P.V only on tiles kept
            f5_exec = f5 / 2 + (f5 / 2) * (1 - skipped / live)
            secondary[label] = {
                "skipped_tiles": skipped, "live_tiles": live,
                "skipped_fraction": round(skipped / live, 6),
                "effective_TFLOPs": round(f5 / m5 / 1e12, 1),
                "executed_TFLOPs": round(f5_exec / m5 / 1e12, 1),
                "ms_per_launch": round(m5 * 1e3, 3),
                "dense_kernel_ms": round(md * 1e3, 3),
                "speedup_vs_dense": round(md / m5, 3),
                "counters": counters("blockskip_s32768" if amp == c5["amplitude"]
                                     else "blockskip_s32768_stress")}
            del q5, k5, v5, o5, l5

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu:
        from oracle import ref_prefill
        from workloads import upcast_f64
        nh = max(1, min(args.cpu_heads, cp["Hq"]))
        nkv = max(1, nh // (cp["Hq"] // cp["Hkv"]))
        qs = upcast_f64(wp.q[:1, :nh])
        ks = upcast_f64(wp.k[:1, :nkv])
        vs = upcast_f64(wp.v[:1, :nkv])
        # repeat the sample until about --cpu-seconds of CPU work has been timed
        reps, t1 = 0, time.perf_counter()
        while True:
            ref_prefill(qs, ks, vs, causal=True, scale=wp.scale)
            reps += 1
            tc = time.perf_counter() - t1
            if tc >= args.cpu_seconds:
                break
        fl = prefill_flops(1, nh, cp["S"], cp["D"], True) * reps
        cores, blas = os.cpu_count(), "unknown"
        try:
            from threadpoolctl import threadpool_info
            info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
            if info:
                cores = max(i.get("num_threads", 1) for i in info)
                blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info}))
        except Exception:
            pass
        cpu = {"value": round(fl / tc / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
               "kind": "oracle", "blas": blas,
               "sample": f"fp64 numpy oracle, {nh} of {cp['Hq']} query heads of the B=1 S=8192 "
                         f"D=128 causal GQA prefill, all rows, run {reps} times; {tc:.2f} s"}

    cnt = counters("gqa_causal_s8192")
    out = {
        "metric": "prefill attention TFLOP/s (% bf16 MFMA peak); paged decode KV GB/s (% HBM)",
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round((pre_s + dec_s) * 1e3, 4),
        "wall_s_timed_region": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V; seeded paged pool)",
        "config": {"workload": "gqa_causal_s8192 prefill (B=1 Hq=32 Hkv=8 S=8192 D=128 causal) "
                               "+ paged_decode_gqa (N=64 L~U[512,4096] Hq=32 Hkv=8 D=128 bs=16)",
                   "global_batch": cp["B"], "seq_len": cp["S"], "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": cnt.get("bytes_per_launch") if cnt else None,
                     "mfma_busy_counter": cnt.get("mfma_busy_frac") if cnt else None,
                     "clock_ghz_counter": cnt.get("clock_ghz") if cnt else None,
                     "kernel": "prefill_bf16_kernel<128,causal>",
                     "us_per_launch": round(pre_s * 1e6, 2), "flops_per_launch": p_flops,
                     "timing": f"HIP events around {args.steps} back-to-back launches"},
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
