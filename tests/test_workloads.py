"""Seeded input generators: determinism, paged-pool round trip, block-table
bijection, the block-skip sink structure.  CPU only."""
import numpy as np
import torch

from workloads import (CONFIGS, blockskip_inputs, decode_inputs, prefill_flops,
                       prefill_inputs, upcast_f64)


def test_prefill_inputs_deterministic_and_rounded():
    a = prefill_inputs(1, 4, 2, 40, 16, seed=7)
    b = prefill_inputs(1, 4, 2, 40, 16, seed=7)
    assert a.q.dtype == torch.bfloat16 and a.k.shape == (1, 2, 40, 16)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    c = prefill_inputs(1, 4, 2, 40, 16, seed=8)
    assert not torch.equal(a.q, c.q)
    # the bf16 tensor is the round-to-nearest-even image of the float32 draw
    rng = np.random.default_rng(7)
    q32 = rng.standard_normal((1, 4, 40, 16), dtype=np.float32)
    bits = q32.view(np.uint32).astype(np.uint64)
    rne = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(a.q.view(torch.int16).numpy().view(np.uint16), rne)


def test_decode_pool_round_trip_and_bijection():
    d = decode_inputs(N=6, Hq=8, Hkv=2, D=8, seed=3, lmin=1, lmax=60, dtype="f32")
    lens = d.seq_lens.numpy()
    nblk = (lens + 15) // 16
    assert d.num_blocks == nblk.sum()
    bt = d.block_table.numpy()
    used = np.concatenate([bt[n, : nblk[n]] for n in range(d.N)])
    assert sorted(used.tolist()) == list(range(d.num_blocks))          # bijection
    assert all((bt[n, nblk[n]:] == -1).all() for n in range(d.N))       # padding
    # regenerating with the same seed reproduces the logical K of sequence 0
    rng = np.random.default_rng(3)
    L = rng.integers(1, 60, size=6, endpoint=True)
    rng.standard_normal((6, 8, 8), dtype=np.float32)
    k0 = rng.standard_normal((int(L[0]), 2, 8), dtype=np.float32)
    kp = d.k_pool.numpy()
    t = np.arange(L[0])
    np.testing.assert_array_equal(kp[bt[0, t // 16], :, t % 16, :], k0)


def test_decode_nan_tails_only_in_unused_slots():
    d = decode_inputs(N=4, Hq=4, Hkv=2, D=8, seed=4, lmin=1, lmax=40, tail="nan", dtype="f32")
    kp = d.k_pool.numpy()
    bt, lens = d.block_table.numpy(), d.seq_lens.numpy()
    for n in range(d.N):
        t = np.arange(lens[n])
        assert np.isfinite(kp[bt[n, t // 16], :, t % 16, :]).all()
    assert np.isnan(kp).sum() == (d.num_blocks * 16 - lens.sum()) * 2 * 8


def test_blockskip_structure():
    w = blockskip_inputs(1, 4, 2, 256, 16, seed=5, amplitude=3.0, n_sinks=8)
    assert len(w.sink_rows) == 8 and len(w.boosted_rows) == 128
    k = upcast_f64(w.k)
    # the boosted coordinate carries about +3 on sink rows, ~N(0,1) elsewhere
    others = np.setdiff1d(np.arange(256), w.sink_rows)
    assert k[0, :, w.sink_rows, w.boost_dim].mean() > 2.0
    assert abs(k[0, :, others, w.boost_dim].mean()) < 0.5


def test_blockskip_split_tiles_halves_disagree():
    """The split-tile input: on every key tile after the first, the first 32
    rows of a 64-row query tile are all negligible (lambda = 1e-3) while the
    last 32 are not, so the tile is kept only through its second half.
    Checked with the decision rule in numpy (float64) on one head."""
    import math
    w = blockskip_inputs(1, 2, 1, 512, 128, seed=7, amplitude=16.0, boosted="split_tiles")
    q = w.q.double().numpy()[0, 0]
    k = w.k.double().numpy()[0, 0]
    ln_lam = math.log(1e-3)
    checked = 0
    for qt in range(1, 8):
        rows = np.arange(qt * 64, qt * 64 + 64)
        s = w.scale * (q[rows] @ k[:(qt + 1) * 64].T)
        s = np.where(np.arange((qt + 1) * 64)[None, :] <= rows[:, None], s, -np.inf)
        tm = s.reshape(64, qt + 1, 64).max(axis=2)
        mp = np.concatenate([np.full((64, 1), -np.inf), np.maximum.accumulate(tm, axis=1)[:, :-1]], axis=1)
        neg = np.isneginf(tm) | (np.isfinite(mp) & (tm - mp < ln_lam))
        for kt in range(1, qt + 1):
            assert neg[:32, kt].all() and not neg[32:, kt].all(), (qt, kt)
            checked += 1
    assert checked == 28


def test_named_configs_and_gqa_saving():
    assert CONFIGS["gqa_causal_s8192"]["Hq"] // CONFIGS["gqa_causal_s8192"]["Hkv"] == 4
    # the GQA page's 32-query-head / 8-group example: the K/V cache shrinks by 75%
    d8 = decode_inputs(N=2, Hq=32, Hkv=8, D=16, seed=1, lens=[10, 20], dtype="f32")
    d32 = decode_inputs(N=2, Hq=32, Hkv=32, D=16, seed=1, lens=[10, 20], dtype="f32")
    assert d8.kv_bytes() * 4 == d32.kv_bytes()
    assert prefill_flops(4, 32, 2048, 128, True) == 4 * 4 * 32 * 128 * 2048 * 2049 // 2
