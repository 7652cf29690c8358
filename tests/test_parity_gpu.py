"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs.

Tolerances (max-abs, on O and on LSE): 2e-2 for bf16 inputs with fp32
accumulation, 1e-4 for float32 inputs.  Block-skip decisions must equal the
oracle's on every tile whose decision margin |gap - ln(lambda)| is at least
1e-3 (the oracle's gap is fp64, the kernel's fp32; tiles inside that margin
are reported, and none occur in the seeded workloads below).
"""
import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as A
from _oracle_pool import oracle_map
from oracle import (ref_blockskip, ref_decode_paged, ref_decode_paged_blockskip, ref_prefill,
                    ref_prefill_paged)
from workloads import (CONFIGS, blockskip_inputs, decode_inputs, paged_prefill_inputs,
                       prefill_inputs, shared_prefix_decode_inputs, unshared_copy, upcast_f64)

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _run_prefill(w):
    dev = "cuda"
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    o, lse = A.prefill(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _compare(o, lse, ro, rl, tol, what):
    eo = float(np.max(np.abs(o.astype(np.float64) - ro)))
    el = float(np.max(np.abs(lse.astype(np.float64) - rl)))
    say(f"{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e} (tol {tol})")
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert eo <= tol, f"{what}: O error {eo}"
    assert el <= tol, f"{what}: LSE error {el}"


# ------------------------------------------------------------------- prefill

def test_tiny_gqa_f32_full():
    c = CONFIGS["tiny_gqa_f32"]
    say("tiny_gqa_f32 B1 Hq4 Hkv2 S128 D64 fp32")
    w = prefill_inputs(c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], seed=c["seed"], dtype="f32")
    o, lse = _run_prefill(w)
    ro, rl = ref_prefill(upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v), causal=True,
                         scale=w.scale)
    _compare(o, lse, ro, rl, TOL["f32"], "tiny_gqa_f32")


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [
    (1, 4, 2, 200, 128, True),     # GQA, ragged tail, several tiles
    (2, 4, 4, 333, 64, True),      # MHA, D=64
    (1, 8, 2, 257, 128, False),    # non-causal GQA
    (1, 8, 1, 130, 128, True),     # MQA
    (1, 16, 2, 300, 128, True),    # group of 8 heads
    (1, 6, 2, 190, 64, True),      # group of 3 heads
    (1, 2, 2, 1, 128, True),       # single token
    (1, 4, 1, 63, 64, False),      # one partial tile
    (1, 4, 4, 513, 128, True),     # MHA, 256-row workgroups + tail
])
def test_prefill_bf16_small(B, Hq, Hkv, S, D, causal):
    say(f"prefill bf16 B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal={causal}")
    w = prefill_inputs(B, Hq, Hkv, S, D, seed=11 + S, causal=causal)
    o, lse = _run_prefill(w)
    ro, rl = ref_prefill(upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v), causal=causal,
                         scale=w.scale)
    _compare(o, lse, ro, rl, TOL["bf16"], "small")


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [
    (1, 8, 2, 2065, 128, True),    # most tiles in the steady-state loop, ragged tail
    (1, 8, 8, 1500, 128, False),   # non-causal MHA, ragged tail
    (2, 8, 8, 1100, 64, True),     # D=64 over many tiles
    (1, 32, 4, 1024, 128, True),   # groups of 8 query heads, 32-row workgroup slices
])
def test_prefill_bf16_medium_all_rows(B, Hq, Hkv, S, D, causal):
    say(f"prefill bf16 medium, every row: B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal={causal}")
    w = prefill_inputs(B, Hq, Hkv, S, D, seed=21 + S, causal=causal)
    o, lse = _run_prefill(w)
    ro, rl = ref_prefill(upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v), causal=causal,
                         scale=w.scale)
    _compare(o, lse, ro, rl, TOL["bf16"], "medium")


@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [
    (8, 64, 64, 300, 128, True),   # 1024 work items: 4 per workgroup
    (27, 19, 19, 500, 64, True),   # 1026 items over 257 workgroups: 3 or 4 each
    (4, 64, 16, 500, 128, False),  # 512 items of 64 rows x 4 heads: 2 per workgroup
    (3, 96, 32, 500, 128, True),   # groups of 3 heads (one head per slot), 576 items: 2 each
    (5, 41, 41, 1100, 64, True),   # 1025 items, odd query-block count, 3 or 4 per workgroup
    (16, 64, 64, 50, 128, True),   # 1024 one-tile items: the ring moves one stage an item
    (16, 64, 64, 100, 64, False),  # 1024 two-tile items, non-causal
])
def test_prefill_bf16_several_items_per_workgroup_all_rows(B, Hq, Hkv, S, D, causal):
    say(f"prefill bf16 several items per workgroup, every row: B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} "
        f"causal={causal}")
    w = prefill_inputs(B, Hq, Hkv, S, D, seed=31 + S, causal=causal)
    o, lse = _run_prefill(w)
    ro, rl = ref_prefill(upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v), causal=causal,
                         scale=w.scale)
    _compare(o, lse, ro, rl, TOL["bf16"], "items")


def test_prefill_f32_variants():
    for (B, Hq, Hkv, S, D, causal) in [(1, 4, 2, 77, 128, True), (2, 2, 1, 50, 64, False)]:
        say(f"prefill f32 B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} causal={causal}")
        w = prefill_inputs(B, Hq, Hkv, S, D, seed=5 + S, causal=causal, dtype="f32")
        o, lse = _run_prefill(w)
        ro, rl = ref_prefill(upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v), causal=causal,
                             scale=w.scale)
        _compare(o, lse, ro, rl, TOL["f32"], "f32")


def _head_jobs(w, **kw):
    """One oracle job per (batch, query head): that head's Q and its group's
    K/V, as float32 (exact for bf16; widened to float64 in the worker)."""
    q, k, v = w.q.float().numpy(), w.k.float().numpy(), w.v.float().numpy()
    G = w.Hq // w.Hkv
    return [((q[b:b + 1, h:h + 1], k[b:b + 1, h // G:h // G + 1], v[b:b + 1, h // G:h // G + 1]),
             dict(scale=w.scale, **kw)) for b in range(w.B) for h in range(w.Hq)]


def _oracle_prefill_all(w, causal):
    """ref_prefill over every (batch, head) and every row, in worker processes."""
    res = oracle_map("ref_prefill", _head_jobs(w, causal=causal))
    ro = np.stack([r[0][0, 0] for r in res]).reshape(w.B, w.Hq, w.S, w.D)
    rl = np.stack([r[1][0, 0] for r in res]).reshape(w.B, w.Hq, w.S)
    return ro, rl


@pytest.mark.parametrize("name", ["mha_causal_s2048", "gqa_causal_s8192"])
def test_prefill_full_size_every_row(name):
    c = CONFIGS[name]
    say(f"{name} full size (the launch the bench times), every row of every head")
    w = prefill_inputs(c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], seed=c["seed"])
    o, lse = _run_prefill(w)
    ro, rl = _oracle_prefill_all(w, True)
    _compare(o, lse, ro, rl, TOL["bf16"], name)


def test_prefill_noncausal_gqa_s8192_every_row():
    say("non-causal GQA B1 Hq32 Hkv8 S8192 D128, every row of every head")
    w = prefill_inputs(1, 32, 8, 8192, 128, seed=1013, causal=False)
    o, lse = _run_prefill(w)
    ro, rl = _oracle_prefill_all(w, False)
    _compare(o, lse, ro, rl, TOL["bf16"], "noncausal s8192")


# -------------------------------------------------------------------- decode

def _run_decode(d, table=None, lens=None, k_pool=None, v_pool=None):
    dev = "cuda"
    q = d.q.to(dev)
    kp = (d.k_pool if k_pool is None else k_pool).to(dev)
    vp = (d.v_pool if v_pool is None else v_pool).to(dev)
    bt = (d.block_table if table is None else table).to(dev)
    sl = (d.seq_lens if lens is None else lens).to(dev)
    o, lse = A.decode_paged(q, kp, vp, bt, sl, d.block_size, d.scale, layout=d.layout)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _ref_decode(d, table=None, lens=None):
    bt = (d.block_table if table is None else table).numpy()
    sl = (d.seq_lens if lens is None else lens).numpy()
    return ref_decode_paged(upcast_f64(d.q), upcast_f64(d.k_pool), upcast_f64(d.v_pool), bt, sl,
                            d.block_size, d.scale, layout=d.layout)


LAYOUTS = ["rowmajor", "mfma"]


@pytest.mark.parametrize("layout", LAYOUTS)
def test_paged_decode_full_config_nan_tails(layout):
    c = CONFIGS["paged_decode_gqa"]
    say(f"paged_decode_gqa full config, NaN-poisoned tail slots, {layout} pools")
    d = decode_inputs(c["N"], c["Hq"], c["Hkv"], c["D"], seed=c["seed"], lmin=c["lmin"],
                      lmax=c["lmax"], tail="nan", layout=layout)
    o, lse = _run_decode(d)
    ro, rl = _ref_decode(d)
    _compare(o, lse, ro, rl, TOL["bf16"], "decode c4")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_paged_decode_permutation_bit_identical(layout):
    say(f"decode: physical block permutation leaves the output bit-identical ({layout})")
    d = decode_inputs(8, 32, 8, 128, seed=77, lmin=1, lmax=700, layout=layout)
    o1, l1 = _run_decode(d)
    perm = torch.from_numpy(np.random.default_rng(78).permutation(d.num_blocks))
    kp2 = torch.empty_like(d.k_pool); kp2[perm] = d.k_pool
    vp2 = torch.empty_like(d.v_pool); vp2[perm] = d.v_pool
    bt = d.block_table.clone()
    m = bt >= 0
    bt[m] = perm[bt[m].long()].to(torch.int32)
    o2, l2 = _run_decode(d, table=bt, k_pool=kp2, v_pool=vp2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ro, rl = _ref_decode(d)
    _compare(o1, l1, ro, rl, TOL["bf16"], "decode perm")


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 128), (16, 1, 64), (8, 4, 64),
                                       (32, 2, 128)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_paged_decode_edge_lengths(Hq, Hkv, D, layout):
    lens = [1, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1000, 0, 1024, 1025, 1537]
    say(f"decode edge lengths Hq{Hq} Hkv{Hkv} D{D} {layout} lens={lens}")
    d = decode_inputs(len(lens), Hq, Hkv, D, seed=90 + D, lens=lens, tail="nan", layout=layout)
    o, lse = _run_decode(d)
    ro, rl = _ref_decode(d)
    z = lens.index(0)
    assert np.all(o[z] == 0) and np.all(np.isneginf(lse[z]))
    keep = [i for i in range(len(lens)) if lens[i] > 0]
    _compare(o[keep], lse[keep], ro[keep], rl[keep], TOL["bf16"], "decode edges")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_paged_decode_bad_table_entries_give_nan(layout):
    say(f"decode: out-of-range table entry and too-long sequence -> NaN rows only ({layout})")
    d = decode_inputs(4, 8, 2, 128, seed=95, lens=[40, 40, 40, 40], layout=layout)
    bt = d.block_table.clone()
    bt[1, 2] = d.num_blocks + 5          # out of range, inside the used blocks
    bt[2, 0] = -7
    lens = d.seq_lens.clone()
    lens[3] = d.max_blocks * 16 + 1      # longer than the table row
    o, lse = _run_decode(d, table=bt, lens=lens)
    assert np.isnan(o[1]).all() and np.isnan(lse[1]).all()
    assert np.isnan(o[2]).all() and np.isnan(o[3]).all()
    ro, rl = _ref_decode(d)
    _compare(o[:1], lse[:1], ro[:1], rl[:1], TOL["bf16"], "decode good row")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_paged_decode_shared_prefix(layout):
    say(f"decode: 8 prompts x 8 samples sharing 1000-token prompts (copy-on-write), {layout}")
    d, _ = shared_prefix_decode_inputs(8, 8, 32, 8, 128, seed=96, prefix_len=1000,
                                       suffix_min=1, suffix_max=600, tail="nan", layout=layout)
    o, lse = _run_decode(d)
    ro, rl = _ref_decode(d)
    _compare(o, lse, ro, rl, TOL["bf16"], "decode shared prefix")
    # the same logical cache without sharing gives the identical bits
    o2, l2 = _run_decode(unshared_copy(d))
    assert np.array_equal(o, o2) and np.array_equal(lse, l2)


# ------------------------------------------------------- chunked paged prefill

def _run_prefill_paged(d):
    o, lse = A.prefill_paged(d.q.cuda(), d.cu_seqlens_q.cuda(), d.k_pool.cuda(), d.v_pool.cuda(),
                             d.block_table.cuda(), d.seq_lens_k.cuda(), d.max_seqlen_q,
                             scale=d.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 128), (16, 2, 64), (8, 1, 128)])
def test_prefill_paged_varlen(Hq, Hkv, D):
    # the last two have 512 and 128 keys: every tile whole, the last included
    ctx = [0, 37, 1000, 5, 300, 0, 64, 448, 0]
    ql = [200, 1, 300, 600, 63, 1, 257, 64, 128]
    say(f"chunked paged prefill Hq{Hq} Hkv{Hkv} D{D} ctx={ctx} q={ql}")
    d = paged_prefill_inputs(ctx, ql, Hq, Hkv, D, seed=120 + D + Hq, tail="nan")
    o, lse = _run_prefill_paged(d)
    ro, rl = ref_prefill_paged(upcast_f64(d.q), d.cu_seqlens_q.numpy(), upcast_f64(d.k_pool),
                               upcast_f64(d.v_pool), d.block_table.numpy(),
                               d.seq_lens_k.numpy(), 16, d.scale)
    _compare(o, lse, ro, rl, TOL["bf16"], "paged prefill")


def test_prefill_paged_bad_device_values_give_nan_rows_only():
    """Malformed device-side descriptions poison only their own rows, with
    bounded writes: a table entry out of the pool (sequence 1), more queries
    than max_seqlen_q (sequence 2), a last query offset past total_q
    (sequence 3).  Guard rows around O and LSE stay untouched; the good
    sequence matches the oracle."""
    say("chunked paged prefill: bad table entry, Sq > max_seqlen_q, cu_seqlens_q past total_q")
    ctx, ql = [100, 50, 200, 30], [40, 64, 100, 20]
    d = paged_prefill_inputs(ctx, ql, 8, 2, 128, seed=140, tail="nan")
    total_q = int(d.cu_seqlens_q[-1])
    cu = d.cu_seqlens_q.clone()
    cu[4] = total_q + 5
    bt = d.block_table.clone()
    bt[1, 2] = d.num_blocks + 3
    G = 7
    o_big = torch.empty((total_q + 2 * G, 8, 128), dtype=torch.bfloat16, device="cuda")
    o_big.view(torch.int16).fill_(0x1234)
    l_big = torch.full((total_q + 2 * G, 8), 123.0, dtype=torch.float32, device="cuda")
    o, lse = o_big[G:G + total_q], l_big[G:G + total_q]
    A.attn_prefill_paged(d.q.cuda(), cu.cuda(), d.k_pool.cuda(), d.v_pool.cuda(), bt.cuda(),
                         d.seq_lens_k.cuda(), o, lse, 64, d.scale)
    torch.cuda.synchronize()
    ob = o_big.view(torch.int16).cpu()
    lb = l_big.cpu()
    assert (ob[:G] == 0x1234).all() and (ob[G + total_q:] == 0x1234).all(), "guard rows of O written"
    assert (lb[:G] == 123.0).all() and (lb[G + total_q:] == 123.0).all(), "guard rows of LSE written"
    of, lf = o.float().cpu().numpy(), lse.cpu().numpy()
    c = d.cu_seqlens_q.numpy()
    for n in (1, 2, 3):
        assert np.isnan(of[c[n]:c[n + 1]]).all() and np.isnan(lf[c[n]:c[n + 1]]).all(), n
    ro, rl = ref_prefill_paged(upcast_f64(d.q), d.cu_seqlens_q.numpy(), upcast_f64(d.k_pool),
                               upcast_f64(d.v_pool), d.block_table.numpy(),
                               d.seq_lens_k.numpy(), 16, d.scale)
    _compare(of[:c[1]], lf[:c[1]], ro[:c[1]], rl[:c[1]], TOL["bf16"], "paged prefill good sequence")


def test_prefill_paged_two_chunks_match_dense_prefill():
    say("two chunks of one sequence through the paged cache = the dense causal prefill")
    S, Hq, Hkv, D = 700, 8, 2, 128
    w = prefill_inputs(1, Hq, Hkv, S, D, seed=131)
    od, ld = _run_prefill(w)                               # [1, Hq, S, D]
    # the same K/V in a paged pool (blocks in order), queries split at 300
    nb = (S + 15) // 16
    kp = torch.zeros((nb, Hkv, 16, D), dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    for j in range(nb):
        t0, t1 = j * 16, min(S, (j + 1) * 16)
        kp[j, :, : t1 - t0] = w.k[0, :, t0:t1]
        vp[j, :, : t1 - t0] = w.v[0, :, t0:t1]
    table = torch.arange(nb, dtype=torch.int32).repeat(2, 1)
    qp = w.q[0].permute(1, 0, 2).contiguous()              # [S, Hq, D]
    cu = torch.tensor([0, 300, 700], dtype=torch.int32)
    seq_k = torch.tensor([300, 700], dtype=torch.int32)    # chunk 1 sees its own 300 keys
    o, lse = A.prefill_paged(qp.cuda(), cu.cuda(), kp.cuda(), vp.cuda(), table.cuda(),
                             seq_k.cuda(), 400, scale=w.scale)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().transpose(1, 0, 2)[None]
    lse = lse.cpu().numpy().T[None]
    _compare(o, lse, od.astype(np.float64), ld.astype(np.float64), TOL["bf16"], "chunks vs dense")


# ---------------------------------------------------------- decode block skip

SPLIT = 512  # tokens per split of the split-KV decode


def _run_decode_skip(d, lam):
    q, kp, vp = d.q.cuda(), d.k_pool.cuda(), d.v_pool.cuda()
    o, lse, bm, cnt = A.decode_paged_blockskip(q, kp, vp, d.block_table.cuda(),
                                               d.seq_lens.cuda(), lam, scale=d.scale,
                                               layout=d.layout)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), bm.cpu().numpy(), int(cnt.item())


def _check_decode_skip(d, lam, what, min_frac=0.0):
    o, lse, bm, cnt = _run_decode_skip(d, lam)
    ro, rl, skip, gap = ref_decode_paged_blockskip(
        upcast_f64(d.q), upcast_f64(d.k_pool), upcast_f64(d.v_pool), d.block_table.numpy(),
        d.seq_lens.numpy(), 16, d.scale, lam=lam, split_tokens=SPLIT, layout=d.layout)
    used = gap > -np.inf
    border = used & (np.abs(gap - math.log(lam)) < 1e-3)
    mism = used & ~border & (bm.astype(bool) != skip)
    say(f"{what}: skipped {int(skip.sum())}/{int(used.sum())} blocks, borderline "
        f"{int(border.sum())}, mismatches {int(mism.sum())}")
    assert mism.sum() == 0
    assert cnt == int(bm[used].astype(np.int64).sum())
    assert skip.sum() >= min_frac * used.sum()
    _compare(o, lse, ro, rl, TOL["bf16"], what)
    return o, lse


@pytest.mark.parametrize("layout", LAYOUTS)
def test_decode_blockskip_stress_decisions(layout):
    say(f"decode block skip: sink stress input, lambda 1e-3 ({layout} pools)")
    d = decode_inputs(16, 32, 8, 128, seed=97, lmin=100, lmax=3000, tail="nan", layout=layout,
                      sink_amplitude=12.0, sink_frac=1 / 64)
    _check_decode_skip(d, 1e-3, f"decode skip stress ({layout})", min_frac=0.2)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_decode_blockskip_tiny_lambda_matches_dense(layout):
    say(f"decode block skip with lambda=1e-30: nothing skipped, equals the dense decode ({layout})")
    d = decode_inputs(8, 32, 8, 128, seed=98, lmin=1, lmax=2000, tail="nan", layout=layout)
    o, lse, bm, cnt = _run_decode_skip(d, 1e-30)
    assert cnt == 0 and bm.sum() == 0
    od, ld = _run_decode(d)
    _compare(o, lse, od.astype(np.float64), ld.astype(np.float64), TOL["bf16"], "skip vs dense")


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 1, 64), (8, 8, 128), (32, 2, 128)])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_decode_blockskip_edge_lengths(Hq, Hkv, D, layout):
    lens = [1, 16, 17, 511, 512, 513, 1000, 0, 1024, 1537]
    say(f"decode block skip edge lengths Hq{Hq} Hkv{Hkv} D{D} ({layout})")
    d = decode_inputs(len(lens), Hq, Hkv, D, seed=99 + D, lens=lens, tail="nan", layout=layout,
                      sink_amplitude=12.0, sink_frac=1 / 32)
    o, lse, bm, cnt = _run_decode_skip(d, 1e-3)
    z = lens.index(0)
    assert np.all(o[z] == 0) and np.all(np.isneginf(lse[z]))
    keep = [i for i in range(len(lens)) if lens[i] > 0]
    dk = dataclasses.replace(d, q=d.q[keep], block_table=d.block_table[keep],
                             seq_lens=d.seq_lens[keep], N=len(keep))
    _check_decode_skip(dk, 1e-3, f"decode skip edges Hq{Hq} Hkv{Hkv} D{D}")


def test_one_rowmajor_cache_serves_prefill_decode_and_skip():
    """One row-major paged cache serves every paged path: the chunked prefill
    with one query per sequence (the query at position L-1 sees all L keys),
    the dense decode and the block-skip decode with a lambda that skips
    nothing give the same rows, and match the oracle."""
    say("one row-major cache: chunked prefill (1 query), dense decode, block-skip decode")
    d = decode_inputs(12, 32, 8, 128, seed=141, lmin=1, lmax=1500, tail="nan", layout="rowmajor")
    od, ld = _run_decode(d)
    os_, ls, bm, cnt = _run_decode_skip(d, 1e-30)
    assert cnt == 0
    N = d.N
    cu = torch.arange(N + 1, dtype=torch.int32)
    op, lp = A.prefill_paged(d.q.cuda(), cu.cuda(), d.k_pool.cuda(), d.v_pool.cuda(),
                             d.block_table.cuda(), d.seq_lens.cuda(), 1, scale=d.scale)
    torch.cuda.synchronize()
    op, lp = op.float().cpu().numpy(), lp.cpu().numpy()
    ro, rl = _ref_decode(d)
    _compare(od, ld, ro, rl, TOL["bf16"], "one cache: decode")
    _compare(os_, ls, ro, rl, TOL["bf16"], "one cache: block-skip decode")
    _compare(op, lp, ro, rl, TOL["bf16"], "one cache: chunked prefill")


# ---------------------------------------------------------------- block skip

def _run_blockskip(w, lam):
    q, k, v = w.q.cuda(), w.k.cuda(), w.v.cuda()
    o, lse, bm, cnt = A.prefill_blockskip(q, k, v, scale=w.scale, lam=lam)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), bm.cpu().numpy(), int(cnt.item())


def _check_decisions(bm, skip, gap, lam, what):
    """Every live tile's decision (kt <= qt) equals the oracle's, except tiles
    whose margin |gap - ln(lambda)| is below 1e-3 (fp64 oracle against fp32
    kernel), which are counted."""
    ln_lam = math.log(lam)
    nT = bm.shape[-1]
    live = np.broadcast_to(np.tril(np.ones((nT, nT), dtype=bool)), skip.shape)
    gpu = bm.astype(bool) & live
    border = live & (np.abs(gap - ln_lam) < 1e-3)
    mism = (gpu != skip) & live & ~border
    say(f"{what}: skipped {int(skip.sum())}/{int(live.sum())} live tiles, "
        f"borderline {int(border.sum())}, mismatches {int(mism.sum())}")
    assert mism.sum() == 0
    return int(border.sum())


def _oracle_blockskip_all(w, lam):
    """ref_blockskip over every (batch, head) and every query tile, in worker
    processes."""
    res = oracle_map("ref_blockskip", _head_jobs(w, lam=lam, tile=64))
    nT = (w.S + 63) // 64
    ro = np.stack([r[0][0, 0] for r in res]).reshape(w.B, w.Hq, w.S, w.D)
    rl = np.stack([r[1][0, 0] for r in res]).reshape(w.B, w.Hq, w.S)
    skip = np.stack([r[2][0, 0] for r in res]).reshape(w.B, w.Hq, nT, nT)
    gap = np.stack([r[3][0, 0] for r in res]).reshape(w.B, w.Hq, nT, nT)
    return ro, rl, skip, gap


def _check_blockskip_all(w, lam, what, min_frac=0.0):
    o, lse, bm, cnt = _run_blockskip(w, lam)
    ro, rl, skip, gap = _oracle_blockskip_all(w, lam)
    _check_decisions(bm, skip, gap, lam, what)
    nT = (w.S + 63) // 64
    live = w.B * w.Hq * nT * (nT + 1) // 2
    assert cnt == int(bm.astype(np.int64).sum())
    assert skip.sum() >= min_frac * live, "the input must exercise the skip path"
    _compare(o, lse, ro, rl, TOL["bf16"], f"{what} O/LSE")
    say(f"{what}: skipped fraction {cnt / live:.6f} ({cnt}/{live})")
    return cnt, live


@pytest.mark.parametrize("B,Hq,Hkv,S,D", [
    (1, 8, 2, 4096, 128),    # groups of 4 heads (the block-skip workload's grouping)
    (1, 8, 8, 2048, 128),    # MHA: one head per workgroup, pairs of adjacent waves
    (1, 6, 3, 2048, 128),    # groups of 2 heads
    (1, 8, 4, 1500, 64),     # D = 64, ragged last tile
    (1, 16, 2, 2048, 128),   # groups of 8 heads, split over two workgroups
    (2, 4, 2, 2048, 128),    # two batches: bitmap rows of batch 1
])
def test_blockskip_stress_full_decisions(B, Hq, Hkv, S, D):
    say(f"block skip stress: B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} amplitude 12, second half boosted")
    w = blockskip_inputs(B, Hq, Hkv, S, D, seed=1105 + S + Hq, amplitude=12.0,
                         boosted="second_half")
    _check_blockskip_all(w, 1e-3, f"stress B{B} Hq{Hq} Hkv{Hkv} S{S} D{D}", min_frac=0.02)


@pytest.mark.parametrize("B,Hq,Hkv,S,D", [
    (1, 8, 2, 2048, 128),    # groups of 4 heads
    (1, 4, 4, 1024, 128),    # one head per K/V group
    (1, 4, 2, 1500, 64),     # D = 64, ragged last tile
])
def test_blockskip_split_tiles(B, Hq, Hkv, S, D):
    """Tiles kept only through their second 32-row half: the wave holding the
    first half skips its exponentials and recomputes the tile a phase later."""
    say(f"block skip split tiles: B{B} Hq{Hq} Hkv{Hkv} S{S} D{D}")
    w = blockskip_inputs(B, Hq, Hkv, S, D, seed=1107 + S, amplitude=16.0, boosted="split_tiles")
    _check_blockskip_all(w, 1e-3, f"split tiles B{B} Hq{Hq} Hkv{Hkv} S{S} D{D}")


def test_blockskip_small_lambda_equals_dense():
    say("block skip with lambda=1e-30 equals the dense kernel")
    w = blockskip_inputs(1, 4, 1, 700, 128, seed=1106, amplitude=12.0, boosted="second_half")
    o, lse, bm, cnt = _run_blockskip(w, 1e-30)
    assert cnt == 0 and bm.sum() == 0
    od, ld = _run_prefill(w)
    assert np.array_equal(o, od) and np.array_equal(lse, ld)


def test_blockskip_full_config_every_tile():
    c = CONFIGS["blockskip_s32768"]
    say("blockskip_s32768 full size: every decision, O and LSE of every head")
    w = blockskip_inputs(c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], seed=c["seed"],
                         amplitude=c["amplitude"], boosted=c["boosted"])
    _check_blockskip_all(w, c["lam"], "blockskip_s32768")


def test_blockskip_full_size_stress_every_tile():
    c = CONFIGS["blockskip_s32768"]
    say("block skip stress at S=32768 (amplitude 12, second half boosted): every decision, "
        "O and LSE of every head")
    w = blockskip_inputs(c["B"], c["Hq"], c["Hkv"], c["S"], c["D"], seed=c["seed"],
                         amplitude=12.0, boosted="second_half")
    _check_blockskip_all(w, c["lam"], "blockskip_s32768 stress", min_frac=0.3)


# ------------------------------------------------------------ FP8 KV decode

def _run_decode_fp8(f, table=None, lens=None, k_pool=None, v_pool=None):
    dev = "cuda"
    b = f.base
    bt = (b.block_table if table is None else table).to(dev)
    sl = (b.seq_lens if lens is None else lens).to(dev)
    kp = (f.k_pool if k_pool is None else k_pool).to(dev)
    vp = (f.v_pool if v_pool is None else v_pool).to(dev)
    o, lse = A.decode_paged_fp8(b.q.to(dev), kp, vp, bt, sl, f.k_scale, f.v_scale,
                                scale=b.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _ref_decode_fp8(f, table=None, lens=None):
    from oracle import ref_decode_paged_fp8
    b = f.base
    bt = (b.block_table if table is None else table).numpy()
    sl = (b.seq_lens if lens is None else lens).numpy()
    return ref_decode_paged_fp8(upcast_f64(b.q), f.k_pool.numpy(), f.v_pool.numpy(), bt, sl, 16,
                                b.scale, f.k_scale, f.v_scale)


def test_paged_decode_fp8_full_config_nan_tails():
    from workloads import fp8_decode_inputs
    c = CONFIGS["paged_decode_gqa"]
    say("paged_decode_gqa full config with FP8 (E4M3) pools, NaN codes in tail slots")
    f = fp8_decode_inputs(c["N"], c["Hq"], c["Hkv"], c["D"], seed=c["seed"], lmin=c["lmin"],
                          lmax=c["lmax"], tail="nan")
    o, lse = _run_decode_fp8(f)
    ro, rl = _ref_decode_fp8(f)
    _compare(o, lse, ro, rl, TOL["bf16"], "decode fp8 c4")


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 128), (16, 1, 64), (8, 4, 64),
                                       (32, 2, 128)])
def test_paged_decode_fp8_edge_lengths(Hq, Hkv, D):
    from workloads import fp8_decode_inputs
    lens = [1, 15, 16, 17, 63, 64, 65, 511, 512, 513, 1000, 0, 1024, 1025, 1537]
    say(f"decode fp8 edge lengths Hq{Hq} Hkv{Hkv} D{D} lens={lens}")
    f = fp8_decode_inputs(len(lens), Hq, Hkv, D, seed=190 + D, lens=lens, tail="nan")
    o, lse = _run_decode_fp8(f)
    ro, rl = _ref_decode_fp8(f)
    z = lens.index(0)
    assert np.all(o[z] == 0) and np.all(np.isneginf(lse[z]))
    keep = [i for i in range(len(lens)) if lens[i] > 0]
    _compare(o[keep], lse[keep], ro[keep], rl[keep], TOL["bf16"], "decode fp8 edges")


def test_paged_decode_fp8_permutation_bit_identical_and_bad_entries():
    from workloads import fp8_decode_inputs
    say("decode fp8: physical block permutation is bit-identical; bad table entries give NaN")
    f = fp8_decode_inputs(8, 32, 8, 128, seed=177, lmin=1, lmax=700)
    o1, l1 = _run_decode_fp8(f)
    b = f.base
    perm = torch.from_numpy(np.random.default_rng(178).permutation(b.num_blocks))
    kp2 = torch.empty_like(f.k_pool); kp2[perm] = f.k_pool
    vp2 = torch.empty_like(f.v_pool); vp2[perm] = f.v_pool
    bt = b.block_table.clone()
    m = bt >= 0
    bt[m] = perm[bt[m].long()].to(torch.int32)
    o2, l2 = _run_decode_fp8(f, table=bt, k_pool=kp2, v_pool=vp2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ro, rl = _ref_decode_fp8(f)
    _compare(o1, l1, ro, rl, TOL["bf16"], "decode fp8 perm")
    bt = b.block_table.clone()
    used = int((bt[1] >= 0).sum())
    bt[1, used - 1] = b.num_blocks + 3
    o3, l3 = _run_decode_fp8(f, table=bt)
    assert np.isnan(o3[1]).all() and np.isnan(l3[1]).all()
    rows = [0] + list(range(2, 8))
    _compare(o3[rows], l3[rows], ro[rows], rl[rows], TOL["bf16"], "decode fp8 good rows")


@pytest.mark.parametrize("layout", LAYOUTS + ["fp8"])
def test_paged_decode_long_sequences_many_splits(layout):
    """Sequences of 9, 18 and 79 splits (the merge's chunked and >64-split paths)."""
    lens = [4097, 9000, 40000]
    say(f"decode long sequences {lens} ({layout})")
    if layout == "fp8":
        from workloads import fp8_decode_inputs
        f = fp8_decode_inputs(3, 16, 4, 128, seed=303, lens=lens, tail="nan")
        o, lse = _run_decode_fp8(f)
        ro, rl = _ref_decode_fp8(f)
    else:
        d = decode_inputs(3, 16, 4, 128, seed=303, lens=lens, tail="nan", layout=layout)
        o, lse = _run_decode(d)
        ro, rl = _ref_decode(d)
    _compare(o, lse, ro, rl, TOL["bf16"], f"decode long ({layout})")
