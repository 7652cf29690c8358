"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]

One step = one pass over the hot path's two entry points: the causal MHA
prefill at the Llama-2-7B attention shape (B=4, Hq=Hkv=32, S=2048, D=128,
bf16) followed by the paged GQA decode (64 sequences, lengths U[512,4096],
Hq=32, Hkv=8, D=128, 16-token blocks).  Inputs are seeded synthetic tensors
already resident in HBM.  W untimed warm-up steps, then exactly K timed steps
bracketed by device synchronisations; each kernel is also timed with HIP
events on the stream it is launched on.  Prints ONE JSON line.

`value` is the prefill throughput in TFLOP/s (algorithmic flops
4*B*Hq*D*S(S+1)/2 over the prefill kernel's mean event time).  The decode
K/V bandwidth, the long-context GQA prefill and the block-skip prefill are
reported under "secondary".  The fp64 CPU oracle is timed on a bounded
sample of the same prefill workload as "cpu_baseline".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
KERNEL_SOURCES = ["prefill_bf16.hip", "decode_paged.hip", "attn_api.cpp", "attn_internal.h"]


def kernel_hash(name: str) -> str:
    p = os.path.join(ROOT, "attention_flash_attn_fwd_amd", "csrc", name)
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    valid only while the kernel source is unchanged since the counters ran."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_sha256_16") != kernel_hash(rec["source"]):
        return None
    return rec.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the GQA-8192 and block-skip measurements")
    ap.add_argument("--cpu-heads", type=int, default=128,
                    help="(batch, head) pairs of the prefill workload the CPU oracle runs")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(no collectives, no sharding); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attention_flash_attn_fwd_amd as A
    from workloads import CONFIGS, blockskip_inputs, decode_inputs, prefill_flops, prefill_inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    A.load()

    # ---------------------------------------------------------------- inputs
    cp = CONFIGS["mha_causal_s2048"]
    wp = prefill_inputs(cp["B"], cp["Hq"], cp["Hkv"], cp["S"], cp["D"], seed=cp["seed"])
    q, k, v = wp.q.to(dev), wp.k.to(dev), wp.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((cp["B"], cp["Hq"], cp["S"]), dtype=torch.float32, device=dev)
    p_flops = prefill_flops(cp["B"], cp["Hq"], cp["S"], cp["D"], True)

    cd = CONFIGS["paged_decode_gqa"]
    wd = decode_inputs(cd["N"], cd["Hq"], cd["Hkv"], cd["D"], seed=cd["seed"], lmin=cd["lmin"],
                       lmax=cd["lmax"], block_size=cd["block_size"], layout="mfma")
    dq = wd.q.to(dev)
    # two copies of the pool, used alternately, so that K/V cannot be served
    # from the 256 MB last-level cache of the previous step
    pools = [(wd.k_pool.to(dev), wd.v_pool.to(dev)) for _ in range(2)]
    dbt, dsl = wd.block_table.to(dev), wd.seq_lens.to(dev)
    do = torch.empty_like(dq)
    dlse = torch.empty((cd["N"], cd["Hq"]), dtype=torch.float32, device=dev)
    ws = torch.empty(A.attn_decode_workspace_bytes(cd["N"], cd["Hq"], cd["D"], wd.max_blocks, 16),
                     dtype=torch.uint8, device=dev)
    kv_bytes = wd.kv_bytes()

    def run_prefill():
        A.attn_prefill(q, k, v, o, lse, True, wp.scale)

    def run_decode(i):
        kp, vp = pools[i % 2]
        A.attn_decode_paged(dq, kp, vp, dbt, dsl, 16, do, dlse, wd.scale, ws, layout="mfma")

    # ------------------------------------------------------------ timed steps
    for i in range(args.warmup):
        run_prefill()
        run_decode(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        e = ev[i]
        e[0].record()
        run_prefill()
        e[1].record()
        e[2].record()
        run_decode(i)
        e[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pre = [e[0].elapsed_time(e[1]) * 1e-3 for e in ev]
    t_dec = [e[2].elapsed_time(e[3]) * 1e-3 for e in ev]
    pre_s = float(np.mean(t_pre))
    dec_s = float(np.mean(t_dec))
    pre_tflops = p_flops / pre_s / 1e12
    dec_gbps = kv_bytes / dec_s / 1e9

    secondary = {
        "paged_decode_gqa": {
            "kv_GBps": round(dec_gbps, 1), "frac_hbm_peak": round(dec_gbps / PEAK_HBM_GBPS, 4),
            "us_per_launch": round(dec_s * 1e6, 2), "us_min": round(min(t_dec) * 1e6, 2),
            "kv_bytes": kv_bytes, "launches": "split + merge", "pool_layout": "mfma",
            "traffic": measured_traffic("decode_native"),
        },
    }

    def time_it(fn, reps, warm=2):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        es = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in es:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) * 1e-3 for a, b in es]
        return float(np.mean(ts)), float(np.min(ts))

    if not args.no_secondary:
        # the same cache in the row-major pool layout (LDS-staged kernel)
        wr = decode_inputs(cd["N"], cd["Hq"], cd["Hkv"], cd["D"], seed=cd["seed"],
                           lmin=cd["lmin"], lmax=cd["lmax"], block_size=cd["block_size"])
        rpools = [(wr.k_pool.to(dev), wr.v_pool.to(dev)) for _ in range(2)]
        ctr = [0]

        def run_rowmajor():
            kp, vp = rpools[ctr[0] % 2]
            ctr[0] += 1
            A.attn_decode_paged(dq, kp, vp, dbt, dsl, 16, do, dlse, wd.scale, ws)
        mr, nr = time_it(run_rowmajor, 20)
        secondary["paged_decode_gqa_rowmajor_pools"] = {
            "kv_GBps": round(kv_bytes / mr / 1e9, 1),
            "frac_hbm_peak": round(kv_bytes / mr / 1e9 / PEAK_HBM_GBPS, 4),
            "us_per_launch": round(mr * 1e6, 2), "us_min": round(nr * 1e6, 2)}
        del rpools

        c3 = CONFIGS["gqa_causal_s8192"]
        w3 = prefill_inputs(c3["B"], c3["Hq"], c3["Hkv"], c3["S"], c3["D"], seed=c3["seed"])
        q3, k3, v3 = w3.q.to(dev), w3.k.to(dev), w3.v.to(dev)
        o3 = torch.empty_like(q3)
        l3 = torch.empty((1, c3["Hq"], c3["S"]), dtype=torch.float32, device=dev)
        m3, n3 = time_it(lambda: A.attn_prefill(q3, k3, v3, o3, l3, True, w3.scale), 10)
        f3 = prefill_flops(1, c3["Hq"], c3["S"], c3["D"], True)
        secondary["gqa_causal_s8192"] = {
            "TFLOPs": round(f3 / m3 / 1e12, 1), "frac_mfma_peak": round(f3 / m3 / 1e12 / PEAK_BF16_TFLOPS, 4),
            "us_per_launch": round(m3 * 1e6, 1)}
        del q3, k3, v3, o3, l3

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
            m5, _ = time_it(lambda: A.attn_prefill_blockskip(q5, k5, v5, o5, l5, w5.scale,
                                                             c5["lam"], 64, None, cnt), 3, warm=1)
            cnt.zero_()
            A.attn_prefill_blockskip(q5, k5, v5, o5, l5, w5.scale, c5["lam"], 64, None, cnt)
            md, _ = time_it(lambda: A.attn_prefill(q5, k5, v5, o5, l5, True, w5.scale), 3, warm=1)
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
                "speedup_vs_dense": round(md / m5, 3)}
            del q5, k5, v5, o5, l5

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu:
        from oracle import ref_prefill
        from workloads import upcast_f64
        nh = max(1, min(args.cpu_heads, cp["B"] * cp["Hq"]))
        qs = upcast_f64(wp.q[:1, :nh])
        ks = upcast_f64(wp.k[:1, :nh])
        vs = upcast_f64(wp.v[:1, :nh])
        t1 = time.perf_counter()
        ref_prefill(qs, ks, vs, causal=True, scale=wp.scale)
        tc = time.perf_counter() - t1
        fl = prefill_flops(1, nh, cp["S"], cp["D"], True)
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
        except Exception:
            cores = os.cpu_count()
        cpu = {"value": round(fl / tc / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
               "kind": "oracle",
               "sample": f"fp64 numpy oracle, {nh} of {cp['B'] * cp['Hq']} (batch, head) pairs of "
                         f"the S=2048 D=128 causal prefill, all rows; {tc:.2f} s"}

    traffic = measured_traffic("prefill_bf16")
    out = {
        "metric": "prefill attention TFLOP/s (% bf16 MFMA peak); paged decode KV GB/s (% HBM)",
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V; seeded paged pool)",
        "config": {"workload": "mha_causal_s2048 prefill (B=4 Hq=Hkv=32 S=2048 D=128 causal) "
                               "+ paged_decode_gqa (N=64 L~U[512,4096] Hq=32 Hkv=8 D=128 bs=16)",
                   "global_batch": cp["B"], "seq_len": cp["S"], "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "prefill_bf16_kernel<128,causal>",
                     "us_per_launch": round(pre_s * 1e6, 2), "us_min": round(min(t_pre) * 1e6, 2),
                     "flops_per_launch": p_flops},
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
