"""Pins for the fp64 oracle: hand-derived worked examples, closed forms,
invariants, an independent library routine and an independent sequential
formulation of block skipping.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (kv_head_of, ref_blockskip, ref_decode_paged, ref_decode_paged_blockskip,
                    ref_prefill, ref_prefill_paged)
from workloads import (decode_inputs, paged_prefill_inputs, shared_prefix_decode_inputs,
                       to_dtype, unshared_copy, upcast_f64)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("causal", [True, False])
def test_golden_causal_ln_weights(causal):
    g = _golden("causal_ln_weights.json")
    q = np.array(g["q"])[None, None]                       # [1,1,3,2]
    k = np.array([[math.log(a), 0.0] for a in g["k_log_args"]])[None, None]
    v = np.array(g["v"])[None, None]
    o, lse = ref_prefill(q, k, v, causal=causal, scale=g["scale"])
    exp = g["causal" if causal else "noncausal"]
    np.testing.assert_allclose(o[0, 0], np.array(exp["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.log(exp["lse_log_args"]), rtol=0, atol=1e-12)


def test_golden_gqa_two_groups():
    g = _golden("gqa_two_groups.json")
    Hq, Hkv, S = 4, 2, 2
    q = np.zeros((1, Hq, S, 1))
    for h, val in enumerate(g["q_heads"]):
        q[0, h, :, 0] = val
    k = np.log(np.array(g["k_heads_log_args"], dtype=np.float64))[None, :, :, None]
    v = np.array(g["v_heads"])[None, :, :, None]
    o, lse = ref_prefill(q, k, v, causal=False, scale=1.0)
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h, :, 0], g["o_heads"][h], atol=1e-12)
        np.testing.assert_allclose(lse[0, h], math.log(g["lse_heads_log_args"][h]), atol=1e-12)


def test_golden_blockskip_sink():
    g = _golden("blockskip_sink.json")
    T = g["tile"]
    k = np.array(g["k"])[None, None, :, None]
    v = np.array(g["v"])[None, None, :, None]
    q = np.ones((1, 1, 4, 1))
    v0, v1, v2, v3 = g["v"]
    for case in g["cases"]:
        o, lse, skip, gap = ref_blockskip(q, k, v, scale=1.0, lam=case["lam"], tile=T)
        assert bool(skip[0, 0, 1, 1]) == case["skip_q1_k1"]
        assert not skip[0, 0, :, 0].any()
        np.testing.assert_allclose(gap[0, 0, 1, 1], -10.0, atol=1e-12)
        e = math.exp(10.0)
        if case["skip_q1_k1"]:
            exp_o = [(v0 + v1) / 2] * 2
            exp_l = [10 + math.log(2)] * 2
        else:
            exp_o = [(e * (v0 + v1) + v2) / (2 * e + 1), (e * (v0 + v1) + v2 + v3) / (2 * e + 2)]
            exp_l = [math.log(2 * e + 1), math.log(2 * e + 2)]
        np.testing.assert_allclose(o[0, 0, 2:, 0], exp_o, rtol=1e-12)
        np.testing.assert_allclose(lse[0, 0, 2:], exp_l, rtol=1e-12)


# --------------------------------------------------------- independent library

@pytest.mark.parametrize("B,Hq,Hkv,S,D,causal", [
    (1, 4, 2, 37, 16, True), (2, 6, 3, 50, 8, False), (1, 8, 1, 33, 32, True),
    (2, 4, 4, 19, 64, True), (1, 4, 2, 128, 64, True),
])
def test_matches_torch_sdpa_fp64(B, Hq, Hkv, S, D, causal):
    """torch's own CPU scaled_dot_product_attention in float64 (its math
    path; GQA via enable_gqa, which repeats each K/V head for consecutive
    query heads) is an independent implementation of the same definition."""
    q = _rand((B, Hq, S, D), 1)
    k = _rand((B, Hkv, S, D), 2)
    v = _rand((B, Hkv, S, D), 3)
    scale = 1.0 / math.sqrt(D) * 1.7
    o, _ = ref_prefill(q, k, v, causal=causal, scale=scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=scale, enable_gqa=True).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ closed forms

def test_causal_row0_is_v0_and_lse_is_score():
    B, Hq, Hkv, S, D = 2, 4, 2, 24, 16
    q, k, v = _rand((B, Hq, S, D), 4), _rand((B, Hkv, S, D), 5), _rand((B, Hkv, S, D), 6)
    scale = 0.3
    o, lse = ref_prefill(q, k, v, causal=True, scale=scale)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            np.testing.assert_allclose(o[b, h, 0], v[b, g, 0], atol=1e-14)
            np.testing.assert_allclose(lse[b, h, 0], scale * q[b, h, 0] @ k[b, g, 0], atol=1e-13)


def test_zero_query_gives_prefix_mean_and_log_count():
    B, Hq, Hkv, S, D = 1, 2, 1, 20, 8
    q = np.zeros((B, Hq, S, D))
    k, v = _rand((B, Hkv, S, D), 7), _rand((B, Hkv, S, D), 8)
    o, lse = ref_prefill(q, k, v, causal=True, scale=1.0)
    for i in range(S):
        np.testing.assert_allclose(o[0, 1, i], v[0, 0, : i + 1].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[0, 1, i], math.log(i + 1), atol=1e-14)
    o, lse = ref_prefill(q, k, v, causal=False, scale=1.0)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0].mean(axis=0), (S, D)), atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], math.log(S), atol=1e-14)


def test_constant_v_gives_constant_output():
    q, k = _rand((1, 4, 30, 16), 9), _rand((1, 2, 30, 16), 10)
    v = np.full((1, 2, 30, 16), -2.75)
    o, _ = ref_prefill(q, k, v, causal=True, scale=0.25)
    np.testing.assert_allclose(o, -2.75, atol=1e-14)


def test_dominant_key_selects_its_value():
    S, D = 12, 4
    q = np.zeros((1, 1, S, D)); q[..., 0] = 1.0
    k = np.zeros((1, 1, S, D)); k[0, 0, 5, 0] = 80.0     # gap of 80 nats
    v = _rand((1, 1, S, D), 11)
    o, lse = ref_prefill(q, k, v, causal=True, scale=1.0)
    np.testing.assert_allclose(o[0, 0, 5:], np.broadcast_to(v[0, 0, 5], (S - 5, D)), atol=1e-15)
    np.testing.assert_allclose(lse[0, 0, 5:], 80.0, atol=1e-12)


# ------------------------------------------------------------------- invariants

def test_identity_values_expose_probabilities():
    """With V = I (D = S) the output rows are the probability rows: they are
    non-negative, sum to 1 and vanish above the diagonal when causal."""
    S = 16
    q, k = _rand((1, 2, S, S), 12), _rand((1, 1, S, S), 13)
    v = np.eye(S)[None, None]
    p, _ = ref_prefill(q, k, v, causal=True, scale=0.5)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)
    assert np.all(np.triu(p[0, 0], 1) == 0) and np.all(np.triu(p[0, 1], 1) == 0)


def test_gqa_equals_mha_on_repeated_kv_and_mqa():
    B, Hq, S, D = 2, 8, 21, 16
    q = _rand((B, Hq, S, D), 14)
    for Hkv in (1, 2, 4, 8):
        k, v = _rand((B, Hkv, S, D), 15 + Hkv), _rand((B, Hkv, S, D), 25 + Hkv)
        o, l = ref_prefill(q, k, v, causal=True, scale=0.2)
        kr = np.repeat(k, Hq // Hkv, axis=1)
        vr = np.repeat(v, Hq // Hkv, axis=1)
        o2, l2 = ref_prefill(q, kr, vr, causal=True, scale=0.2)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(l, l2)
    assert [kv_head_of(h, 32, 8) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]


def test_noncausal_key_permutation_invariance():
    q, k, v = _rand((1, 2, 25, 8), 30), _rand((1, 2, 25, 8), 31), _rand((1, 2, 25, 8), 32)
    perm = np.random.default_rng(33).permutation(25)
    o, l = ref_prefill(q, k, v, causal=False, scale=0.7)
    o2, l2 = ref_prefill(q, k[:, :, perm], v[:, :, perm], causal=False, scale=0.7)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(l, l2, atol=1e-13)


def test_lse_merge_over_key_partition():
    """The log-sum-exp of the whole row equals ln(sum_s exp(lse_s)) over any
    partition of the keys into parts, and O is the exp(lse_s - lse)-weighted
    sum of the parts' outputs (the identity split-KV decoding relies on)."""
    rng = np.random.default_rng(40)
    L, D, Hq, Hkv = 57, 16, 4, 2
    q = rng.standard_normal((1, Hq, L, D)); k = rng.standard_normal((1, Hkv, L, D))
    v = rng.standard_normal((1, Hkv, L, D))
    o, lse = ref_prefill(q, k, v, causal=False, scale=0.4)
    cuts = np.sort(rng.choice(np.arange(1, L), size=3, replace=False))
    parts = np.split(np.arange(L), cuts)
    os_, ls_ = [], []
    for idx in parts:
        # a part is attention restricted to its keys (non-causal)
        op, lp = ref_prefill(q[:, :, : len(idx)] * 0 + q[:, :, :1], k[:, :, idx], v[:, :, idx],
                             causal=False, scale=0.4)
        os_.append(op[:, :, 0]); ls_.append(lp[:, :, 0])
    ls_ = np.stack(ls_)                       # [parts, 1, Hq]
    tot = np.log(np.sum(np.exp(ls_), axis=0))
    np.testing.assert_allclose(tot, lse[:, :, 0], atol=1e-13)
    w = np.exp(ls_ - tot)[..., None]
    np.testing.assert_allclose(np.sum(w * np.stack(os_), axis=0), o[:, :, 0], atol=1e-13)


# ----------------------------------------------------------------------- decode

def _decode_small(tail="zero", seed=50, N=5):
    return decode_inputs(N=N, Hq=8, Hkv=2, D=16, seed=seed, lmin=1, lmax=70, block_size=16,
                         tail=tail, dtype="f32")


def test_decode_equals_last_prefill_row():
    d = _decode_small()
    q, kp, vp = upcast_f64(d.q), upcast_f64(d.k_pool), upcast_f64(d.v_pool)
    o, lse = ref_decode_paged(q, kp, vp, d.block_table.numpy(), d.seq_lens.numpy(),
                              d.block_size, d.scale)
    for n in range(d.N):
        L = int(d.seq_lens[n])
        t = np.arange(L)
        phys = d.block_table.numpy()[n, t // 16]
        kl = kp[phys, :, t % 16, :].transpose(1, 0, 2)[None]     # [1,Hkv,L,D]
        vl = vp[phys, :, t % 16, :].transpose(1, 0, 2)[None]
        qq = np.zeros((1, d.Hq, L, d.D)); qq[0, :, L - 1] = q[n]
        op, lp = ref_prefill(qq, kl, vl, causal=True, scale=d.scale, rows=[L - 1])
        np.testing.assert_allclose(o[n], op[0, :, 0], atol=1e-13)
        np.testing.assert_allclose(lse[n], lp[0, :, 0], atol=1e-13)


def test_decode_invariant_under_physical_permutation_and_nan_tails():
    d = _decode_small(tail="nan")
    q, kp, vp = upcast_f64(d.q), upcast_f64(d.k_pool), upcast_f64(d.v_pool)
    bt = d.block_table.numpy()
    o, lse = ref_decode_paged(q, kp, vp, bt, d.seq_lens.numpy(), 16, d.scale)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    perm = np.random.default_rng(51).permutation(kp.shape[0])   # old -> new position
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm], vp2[perm] = kp, vp
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1)
    o2, lse2 = ref_decode_paged(q, kp2, vp2, bt2, d.seq_lens.numpy(), 16, d.scale)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_decode_empty_sequence():
    d = decode_inputs(N=3, Hq=4, Hkv=2, D=8, seed=52, lens=[0, 5, 17], dtype="f32")
    o, lse = ref_decode_paged(upcast_f64(d.q), upcast_f64(d.k_pool), upcast_f64(d.v_pool),
                              d.block_table.numpy(), d.seq_lens.numpy(), 16, d.scale)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.isfinite(o[1:]).all()


@pytest.mark.parametrize("layout", ["rowmajor", "mfma"])
def test_shared_prefix_cache(layout):
    """Copy-on-write sharing (PageAttention part of the KV-cache survey page):
    the samples of a prompt alias the prompt's full blocks, own a copy of its
    partly filled last block, and read exactly the logical sequence they
    would read from an unshared cache."""
    P, M, Lp = 3, 4, 37
    d, logical = shared_prefix_decode_inputs(P, M, 8, 2, 16, seed=53, prefix_len=Lp,
                                             suffix_min=1, suffix_max=40, dtype="f32",
                                             tail="nan", layout=layout)
    bt = d.block_table.numpy()
    ns = Lp // 16
    for p_ in range(P):
        rows = bt[p_ * M:(p_ + 1) * M]
        assert (rows[:, :ns] == rows[0, :ns]).all()             # aliased prompt blocks
        assert len(set(rows[:, ns].tolist())) == M              # one private copy each
    private = [int(x) for n in range(d.N) for x in bt[n, ns:] if x >= 0]
    assert len(private) == len(set(private))
    assert d.num_blocks < unshared_copy(d).num_blocks
    args = (upcast_f64(d.q),)
    o, lse = ref_decode_paged(*args, upcast_f64(d.k_pool), upcast_f64(d.v_pool), bt,
                              d.seq_lens.numpy(), 16, d.scale, layout=layout)
    u = unshared_copy(d)
    o2, lse2 = ref_decode_paged(*args, upcast_f64(u.k_pool), upcast_f64(u.v_pool),
                                u.block_table.numpy(), u.seq_lens.numpy(), 16, d.scale,
                                layout=layout)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)
    # each sequence: the last causal row of a prefill over its logical K/V
    for n in range(d.N):
        K, V = (upcast_f64(to_dtype(x, "f32")) for x in logical[n])
        L = K.shape[0]
        qq = np.zeros((1, d.Hq, L, d.D)); qq[0, :, L - 1] = args[0][n]
        op, lp = ref_prefill(qq, K.transpose(1, 0, 2)[None], V.transpose(1, 0, 2)[None],
                             causal=True, scale=d.scale, rows=[L - 1])
        np.testing.assert_allclose(o[n], op[0, :, 0], atol=1e-13)
        np.testing.assert_allclose(lse[n], lp[0, :, 0], atol=1e-13)


# ------------------------------------------------------- chunked paged prefill

def _logical_kv(ctx, ql, Hq, Hkv, D, seed):
    """Re-draw the generator's logical K/V (documented draw order: packed q,
    then per sequence K then V), independent of the pool and the table."""
    rng = np.random.default_rng(seed)
    rng.standard_normal((int(sum(ql)), Hq, D), dtype=np.float32)
    out = []
    for c, qn in zip(ctx, ql):
        L = c + qn
        k = rng.standard_normal((L, Hkv, D), dtype=np.float32)
        v = rng.standard_normal((L, Hkv, D), dtype=np.float32)
        out.append((upcast_f64(to_dtype(k, "f32")), upcast_f64(to_dtype(v, "f32"))))
    return out


@pytest.mark.parametrize("layout", ["rowmajor", "mfma"])
def test_paged_prefill_chunks_are_rows_of_the_full_prefill(layout):
    ctx, ql = [0, 37, 100, 5], [20, 1, 70, 33]
    d = paged_prefill_inputs(ctx, ql, 4, 2, 16, seed=61, dtype="f32", tail="nan", layout=layout)
    q = upcast_f64(d.q)
    o, lse = ref_prefill_paged(q, d.cu_seqlens_q.numpy(), upcast_f64(d.k_pool),
                               upcast_f64(d.v_pool), d.block_table.numpy(),
                               d.seq_lens_k.numpy(), 16, d.scale, layout=layout)
    cu = d.cu_seqlens_q.numpy()
    for n, (K, V) in enumerate(_logical_kv(ctx, ql, 4, 2, 16, 61)):
        L = K.shape[0]
        qq = np.zeros((1, 4, L, 16))
        qq[0, :, ctx[n]:] = q[cu[n]:cu[n + 1]].transpose(1, 0, 2)
        rows = np.arange(ctx[n], L)
        of, lf = ref_prefill(qq, K.transpose(1, 0, 2)[None], V.transpose(1, 0, 2)[None],
                             causal=True, scale=d.scale, rows=rows)
        np.testing.assert_allclose(o[cu[n]:cu[n + 1]], of[0].transpose(1, 0, 2), atol=1e-13)
        np.testing.assert_allclose(lse[cu[n]:cu[n + 1]], lf[0].T, atol=1e-13)


def test_paged_prefill_single_token_chunk_is_decode():
    ctx = [3, 50, 200]
    d = paged_prefill_inputs(ctx, [1, 1, 1], 8, 2, 16, seed=62, dtype="f32")
    args = (upcast_f64(d.k_pool), upcast_f64(d.v_pool), d.block_table.numpy())
    o, lse = ref_prefill_paged(upcast_f64(d.q), d.cu_seqlens_q.numpy(), *args,
                               d.seq_lens_k.numpy(), 16, d.scale)
    od, ld = ref_decode_paged(upcast_f64(d.q), *args, d.seq_lens_k.numpy(), 16, d.scale)
    np.testing.assert_allclose(o, od, atol=1e-13)
    np.testing.assert_allclose(lse, ld, atol=1e-13)


def test_paged_prefill_brute_force_tiny():
    ctx, ql = [2, 0], [3, 2]
    d = paged_prefill_inputs(ctx, ql, 2, 1, 4, seed=63, dtype="f32", block_size=16)
    q = upcast_f64(d.q)
    o, _ = ref_prefill_paged(q, d.cu_seqlens_q.numpy(), upcast_f64(d.k_pool),
                             upcast_f64(d.v_pool), d.block_table.numpy(), d.seq_lens_k.numpy(),
                             16, d.scale)
    logical = _logical_kv(ctx, ql, 2, 1, 4, 63)
    r = 0
    for n in range(2):
        K, V = logical[n]
        for i in range(ql[n]):
            pos = ctx[n] + i
            for h in range(2):
                w = [math.exp(d.scale * sum(q[r, h, x] * K[j, 0, x] for x in range(4)))
                     for j in range(pos + 1)]
                z = sum(w)
                for x in range(4):
                    ref = sum(w[j] * V[j, 0, x] for j in range(pos + 1)) / z
                    assert abs(o[r, h, x] - ref) < 1e-12
            r += 1


# ------------------------------------------------------------ decode block skip

def _decode_skip_replay(q, kp, vp, bt, lens, bs, scale, lam, split):
    """Decode block skipping replayed block by block: per (sequence, K/V
    head, split), a running max per query head over the KEPT blocks only,
    each block tested before it is folded in; outputs from the kept tokens
    with explicit loops.  Independent of the prefix-max formulation."""
    N, Hq, D = q.shape
    Hkv = kp.shape[1]
    G = Hq // Hkv
    ln_lam = math.log(lam)
    out = np.zeros((N, Hq, D))
    skip = np.zeros((N, Hkv, bt.shape[1]), dtype=bool)
    for n in range(N):
        L = int(lens[n])
        for g in range(Hkv):
            kept = []
            for s0 in range(0, L, split):
                m = np.full(G, -np.inf)
                for b in range(s0 // bs, (min(L, s0 + split) + bs - 1) // bs):
                    toks = list(range(b * bs, min(L, (b + 1) * bs)))
                    rows = np.array([kp[bt[n, t // bs], g, t % bs] for t in toks])
                    tm = np.array([max(scale * float(q[n, g * G + h] @ r) for r in rows)
                                   for h in range(G)])
                    if np.all(np.isfinite(m)) and np.all(tm - m < ln_lam):
                        skip[n, g, b] = True
                        continue
                    m = np.maximum(m, tm)
                    kept += toks
            for h in range(g * G, (g + 1) * G):
                sc = np.array([scale * float(q[n, h] @ kp[bt[n, t // bs], g, t % bs]) for t in kept])
                w = np.exp(sc - sc.max())
                w /= w.sum()
                out[n, h] = sum(wi * vp[bt[n, t // bs], g, t % bs] for wi, t in zip(w, kept))
    return out, skip


@pytest.mark.parametrize("lam,amp,frac", [(1e-3, 12.0, 1 / 64), (1e-2, 6.0, 1 / 16),
                                          (1e-3, 0.0, 0.0)])
def test_decode_blockskip_prefix_max_equals_replay(lam, amp, frac):
    d = decode_inputs(N=3, Hq=4, Hkv=2, D=16, seed=57, lmin=60, lmax=200, dtype="f32",
                      sink_amplitude=amp, sink_frac=frac)
    q, kp, vp = upcast_f64(d.q), upcast_f64(d.k_pool), upcast_f64(d.v_pool)
    bt, lens = d.block_table.numpy(), d.seq_lens.numpy()
    o, lse, skip, gap = ref_decode_paged_blockskip(q, kp, vp, bt, lens, 16, d.scale, lam=lam,
                                                   split_tokens=64)
    ro, rskip = _decode_skip_replay(q, kp, vp, bt, lens, 16, d.scale, lam, 64)
    np.testing.assert_array_equal(skip, rskip)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    used = gap > -np.inf
    assert np.array_equal(skip[used], gap[used] < math.log(lam)) and not skip[~used].any()
    if amp:
        assert skip.sum() > 0
    # never the first block of a split
    assert not skip[:, :, ::4].any()


def test_decode_blockskip_tiny_lambda_and_error_bound():
    d = decode_inputs(N=4, Hq=8, Hkv=2, D=32, seed=58, lmin=100, lmax=700, dtype="f32",
                      sink_amplitude=10.0, sink_frac=1 / 50)
    args = (upcast_f64(d.q), upcast_f64(d.k_pool), upcast_f64(d.v_pool), d.block_table.numpy(),
            d.seq_lens.numpy(), 16, d.scale)
    o0, l0 = ref_decode_paged(*args)
    o1, l1, skip, _ = ref_decode_paged_blockskip(*args, lam=1e-300, split_tokens=256)
    assert not skip.any()
    np.testing.assert_allclose(o1, o0, atol=1e-13)      # same sums, other order
    np.testing.assert_allclose(l1, l0, atol=1e-13)
    o2, l2, skip, _ = ref_decode_paged_blockskip(*args, lam=1e-3, split_tokens=256)
    assert skip.sum() > 0
    # error bound: the dropped softmax mass, times 2 max|V|
    dropped = 1.0 - np.exp(l2 - l0)
    vmax = np.abs(upcast_f64(d.v_pool)).max()
    assert np.all(np.abs(o2 - o0).max(axis=2) <= 2 * vmax * dropped + 1e-12)
    assert dropped.max() < 1e-2


# -------------------------------------------------------------------- blockskip

def _sequential_blockskip(q, k, v, scale, lam, T):
    """The online algorithm replayed tile by tile for one head: a running
    max m and sum l per row, key tiles in ascending order, each tile's row
    maxima tested against m BEFORE the tile is folded in; skipped tiles are
    not folded in at all.  Independent of the prefix-max formulation."""
    S, D = q.shape
    ln_lam = math.log(lam)
    nT = (S + T - 1) // T
    O = np.zeros((S, D)); LSE = np.zeros(S)
    skip = np.zeros((nT, nT), dtype=bool)
    for qt in range(nT):
        rows = np.arange(qt * T, min(S, (qt + 1) * T))
        m = np.full(len(rows), -np.inf); l = np.zeros(len(rows)); acc = np.zeros((len(rows), D))
        for kt in range(qt + 1):
            cols = np.arange(kt * T, min(S, (kt + 1) * T))
            s = scale * q[rows] @ k[cols].T
            s[cols[None, :] > rows[:, None]] = -np.inf
            tm = s.max(axis=1)
            with np.errstate(invalid="ignore"):
                neg = np.isneginf(tm) | (np.isfinite(m) & (tm - m < ln_lam))
            if neg.all():
                skip[qt, kt] = True
                continue
            m_new = np.maximum(m, tm)
            alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
            p = np.exp(s - m_new[:, None])
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[cols]
            m = m_new
        O[rows] = acc / l[:, None]
        LSE[rows] = m + np.log(l)
    return O, LSE, skip


@pytest.mark.parametrize("S,amp,lam", [(96, 12.0, 1e-3), (128, 12.0, 1e-2), (80, 3.0, 1e-3),
                                       (150, 20.0, 0.3)])
def test_blockskip_prefix_max_equals_sequential_replay(S, amp, lam):
    from workloads import blockskip_inputs
    T = 16
    w = blockskip_inputs(1, 2, 1, S, 16, seed=60, amplitude=amp, n_sinks=4,
                         boosted="second_half", dtype="f32", scale=0.25)
    q, k, v = upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v)
    o, lse, skip, _ = ref_blockskip(q, k, v, scale=w.scale, lam=lam, tile=T)
    for h in range(2):
        so, sl, ss = _sequential_blockskip(q[0, h], k[0, 0], v[0, 0], w.scale, lam, T)
        np.testing.assert_array_equal(skip[0, h], ss)
        np.testing.assert_allclose(o[0, h], so, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], sl, atol=1e-12)
    if amp >= 12:
        assert skip.any(), "stress inputs must exercise the skip path"


def test_blockskip_tiny_lambda_is_exact_attention_and_error_bound():
    from workloads import blockskip_inputs
    w = blockskip_inputs(1, 2, 1, 128, 16, seed=61, amplitude=12.0, n_sinks=4,
                         boosted="second_half", dtype="f32", scale=0.25)
    q, k, v = upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v)
    o_ex, l_ex = ref_prefill(q, k, v, causal=True, scale=w.scale)
    o0, l0, s0, _ = ref_blockskip(q, k, v, scale=w.scale, lam=1e-300, tile=16)
    assert not s0.any()
    np.testing.assert_allclose(o0, o_ex, atol=1e-13)
    np.testing.assert_allclose(l0, l_ex, atol=1e-13)
    o1, l1, s1, _ = ref_blockskip(q, k, v, scale=w.scale, lam=1e-3, tile=16)
    assert s1.any()
    # dropped probability mass per row: 1 - exp(LSE_kept - LSE_full); the
    # output moves by at most 2 * max|V| times that mass
    mass = 1.0 - np.exp(l1 - l_ex)
    err = np.abs(o1 - o_ex).max(axis=-1)
    assert np.all(err <= 2 * np.abs(v).max() * mass + 1e-12)
    assert np.all(l1 <= l_ex + 1e-13)


def test_blockskip_qtile_subset_matches_full():
    from workloads import blockskip_inputs
    w = blockskip_inputs(1, 4, 2, 96, 8, seed=62, amplitude=12.0, n_sinks=3,
                         boosted="second_half", dtype="f32", scale=0.35)
    q, k, v = upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v)
    o, l, s, g = ref_blockskip(q, k, v, scale=w.scale, lam=1e-3, tile=16)
    sel = [1, 4, 5]
    o2, l2, s2, g2 = ref_blockskip(q, k, v, scale=w.scale, lam=1e-3, tile=16, qtiles=sel)
    rows = np.concatenate([np.arange(t * 16, (t + 1) * 16) for t in sel])
    np.testing.assert_array_equal(o[:, :, rows], o2)
    np.testing.assert_array_equal(s[:, :, sel], s2)


def test_decode_layouts_hold_the_same_cache():
    """The two pool layouts are index permutations of the same cache: the
    generator draws identical values and the oracle gives identical results;
    element checks pin both layout definitions."""
    from oracle import pool_rows
    a = decode_inputs(N=3, Hq=8, Hkv=2, D=16, seed=70, lmin=1, lmax=40, dtype="f32")
    b = decode_inputs(N=3, Hq=8, Hkv=2, D=16, seed=70, lmin=1, lmax=40, dtype="f32", layout="mfma")
    assert b.k_pool.shape == (a.num_blocks, 2, 2, 16, 8) and b.v_pool.shape == (a.num_blocks, 2, 16, 16)
    ka, kb = a.k_pool.numpy(), b.k_pool.numpy()
    va, vb = a.v_pool.numpy(), b.v_pool.numpy()
    # K element (block p, head g, token t, dim d) sits at chunk d // 8, slot d % 8
    assert kb[1, 1, 1, 5, 2] == ka[1, 1, 5, 8 + 2]
    assert vb[2, 0, 7, 9] == va[2, 0, 9, 7]                 # V transposed in the block
    np.testing.assert_array_equal(pool_rows(kb, "mfma", "k"), ka)
    np.testing.assert_array_equal(pool_rows(vb, "mfma", "v"), va)
    oa = ref_decode_paged(upcast_f64(a.q), upcast_f64(a.k_pool), upcast_f64(a.v_pool),
                          a.block_table.numpy(), a.seq_lens.numpy(), 16, a.scale)
    ob = ref_decode_paged(upcast_f64(b.q), upcast_f64(b.k_pool), upcast_f64(b.v_pool),
                          b.block_table.numpy(), b.seq_lens.numpy(), 16, b.scale, layout="mfma")
    np.testing.assert_array_equal(oa[0], ob[0])
    np.testing.assert_array_equal(oa[1], ob[1])


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV cache

def test_fp8_code_values_match_torch_and_closed_forms():
    """The E4M3 table written from the format definition equals torch's own
    float8_e4m3fn decoding on all 256 codes (NaN where torch has NaN), and
    hits the format's landmark values."""
    from oracle import fp8_e4m3_value
    v = fp8_e4m3_value(np.arange(256))
    t = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(v, t)                      # NaNs compare equal here
    assert v[0x38] == 1.0 and v[0x30] == 0.5 and v[0x3C] == 1.5
    assert v[0x7E] == 448.0                                  # largest finite
    assert v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9  # subnormals
    assert v[0x08] == 2.0 ** -6                              # smallest normal
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                           # codes 0..126 increase
    np.testing.assert_array_equal(v[0x80:0xFF], -pos)         # sign bit


def test_fp8_pool_byte_order_and_dequantized_decode():
    """The oracle's reading of the FP8 pool byte order inverts the
    generator's (written separately, as reshapes), a few bytes sit where the
    layout definition puts them, and the FP8 decode equals the plain decode
    on the pools dequantized by torch."""
    from oracle import fp8_pool_rows, ref_decode_paged_fp8
    from workloads import fp8_decode_inputs
    f = fp8_decode_inputs(N=3, Hq=8, Hkv=2, D=128, seed=71, lens=[17, 1, 40], tail="nan")
    b = f.base
    kp, vp = f.k_pool.numpy(), f.v_pool.numpy()
    kc, vc = f.k_codes.numpy(), f.v_codes.numpy()
    np.testing.assert_array_equal(fp8_pool_rows(kp, "k", 128), kc)
    np.testing.assert_array_equal(fp8_pool_rows(vp, "v", 128), vc)
    # K (token 3, dim 5*16+2): chunk 5 -> run byte 1024 + (1*16 + 3)*16 + 2
    assert kp[1, 1, 1024 + 19 * 16 + 2] == kc[1, 1, 3, 82]
    # V (token 6, dim 6*16+9): group 1, block 6 -> 1024 + (1*16 + 9)*16 + 2*4 + 2
    assert vp[2, 0, 1024 + 25 * 16 + 8 + 2] == vc[2, 0, 6, 105]
    args = (b.block_table.numpy(), b.seq_lens.numpy(), 16, b.scale)
    q = upcast_f64(b.q)
    o, l = ref_decode_paged_fp8(q, kp, vp, *args, f.k_scale, f.v_scale)
    o2, l2 = ref_decode_paged(q, f.k_rows.numpy(), f.v_rows.numpy(), *args)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    assert np.isfinite(o).all()                               # NaN tail codes never read


def test_fp8_decode_within_quantisation_bound():
    """Against the plain decode on the unquantised bf16 pools, the FP8
    decode stays inside the bound that E4M3 rounding allows: with
    dV = max |v_hat - v| and E = scale * max_j sum_d |q_d| |k_hat_jd - k_jd|,
    |O_hat - O| <= dV + (exp(2E) - 1) max |v_hat|  and  |LSE_hat - LSE| <= E.
    A wrong scale, byte order or code value breaks it at once."""
    from oracle import ref_decode_paged_fp8
    from workloads import fp8_decode_inputs
    f = fp8_decode_inputs(N=4, Hq=8, Hkv=2, D=64, seed=72, lmin=1, lmax=300)
    b = f.base
    q = upcast_f64(b.q)
    table, lens = b.block_table.numpy(), b.seq_lens.numpy()
    o, l = ref_decode_paged_fp8(q, f.k_pool.numpy(), f.v_pool.numpy(), table, lens, 16, b.scale,
                                f.k_scale, f.v_scale)
    k, v = upcast_f64(b.k_pool), upcast_f64(b.v_pool)
    o_ref, l_ref = ref_decode_paged(q, k, v, table, lens, 16, b.scale)
    kh, vh = f.k_rows.numpy(), f.v_rows.numpy()
    # the E4M3 rounding itself: relative 2^-4 (normal), absolute 2^-10 * scale (subnormal)
    assert np.all(np.abs(kh - k) <= np.maximum(2.0 ** -4 * np.abs(k), 2.0 ** -10 * f.k_scale) + 1e-15)
    for n in range(b.N):
        L = int(lens[n])
        t = np.arange(L)
        ph, sl = table[n, t // 16], t % 16
        for h in range(b.Hq):
            g = h // (b.Hq // b.Hkv)
            dk = np.abs(kh[ph, g, sl] - k[ph, g, sl])          # [L, D]
            dv = np.abs(vh[ph, g, sl] - v[ph, g, sl]).max()
            E = b.scale * (dk @ np.abs(q[n, h])).max()
            bound = dv + math.expm1(2 * E) * np.abs(vh[ph, g, sl]).max()
            assert np.abs(o[n, h] - o_ref[n, h]).max() <= bound + 1e-12
            assert abs(l[n, h] - l_ref[n, h]) <= E + 1e-12
    # and the bound is not vacuous: the quantised result is close
    assert np.abs(o - o_ref).max() < 0.25


def test_oracle_pool_equals_direct_calls():
    """The worker pool the full-size GPU tests use returns exactly what the
    oracle returns when called directly (float32 inputs widened exactly)."""
    from _oracle_pool import oracle_map
    from workloads import blockskip_inputs
    w = blockskip_inputs(1, 4, 2, 200, 16, seed=64, amplitude=12.0, n_sinks=3,
                         boosted="second_half", scale=0.3)
    q, k, v = w.q.float().numpy(), w.k.float().numpy(), w.v.float().numpy()
    jobs = [((q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1]),
             dict(scale=w.scale, lam=1e-3, tile=64)) for h in range(4)]
    res = oracle_map("ref_blockskip", jobs)
    full = ref_blockskip(upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v), scale=w.scale,
                         lam=1e-3, tile=64)
    for h in range(4):
        for i in range(4):
            np.testing.assert_array_equal(res[h][i][0, 0], full[i][0, h])
    res = oracle_map("ref_prefill", [(a, dict(scale=w.scale, causal=True)) for a, _ in jobs])
    o, l = ref_prefill(upcast_f64(w.q), upcast_f64(w.k), upcast_f64(w.v), causal=True,
                       scale=w.scale)
    for h in range(4):
        np.testing.assert_array_equal(res[h][0][0, 0], o[0, h])
        np.testing.assert_array_equal(res[h][1][0, 0], l[0, h])
