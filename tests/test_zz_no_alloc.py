"""The allocation-free paged decode (attn_decode_paged_noalloc) against the
workspace decode (attn_decode_paged) through the C ABI: the same kernels run,
so the outputs must be bit-identical, and both must match the fp64 oracle
within the bf16 tolerance.  Two calls in a row share the library's static
scratch; the second, smaller one must not see the first one's contents.
"""
import sys

import numpy as np
import pytest
import torch

import attention_flash_attn_fwd_amd as A
from oracle import ref_decode_paged
from workloads import CONFIGS, decode_inputs, upcast_f64

pytestmark = pytest.mark.gpu

TOL = 2e-2


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _both(d):
    q, kp, vp = d.q.cuda(), d.k_pool.cuda(), d.v_pool.cuda()
    bt, sl = d.block_table.cuda(), d.seq_lens.cuda()
    o1, l1 = A.decode_paged_noalloc(q, kp, vp, bt, sl, 16, d.scale, layout=d.layout)
    torch.cuda.synchronize()
    o1, l1 = o1.float().cpu().numpy(), l1.cpu().numpy()
    o2, l2 = A.decode_paged(q, kp, vp, bt, sl, 16, d.scale, layout=d.layout)
    torch.cuda.synchronize()
    return o1, l1, o2.float().cpu().numpy(), l2.cpu().numpy()


def test_noalloc_decode_two_calls_match_workspace_decode():
    c = CONFIGS["paged_decode_gqa"]
    cases = [
        ("decode workload, 64 sequences, row-major pools",
         dict(N=c["N"], Hq=c["Hq"], Hkv=c["Hkv"], D=c["D"], seed=c["seed"], lmin=c["lmin"],
              lmax=c["lmax"], layout="rowmajor")),
        ("smaller second call, 8 sequences of 1..700 tokens, MFMA-native pools",
         dict(N=8, Hq=32, Hkv=8, D=128, seed=77, lmin=1, lmax=700, layout="mfma")),
    ]
    for what, kw in cases:
        say(f"noalloc decode: {what}")
        d = decode_inputs(kw["N"], kw["Hq"], kw["Hkv"], kw["D"], seed=kw["seed"],
                          lmin=kw["lmin"], lmax=kw["lmax"], tail="nan", layout=kw["layout"])
        o1, l1, o2, l2 = _both(d)
        assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)
        ro, rl = ref_decode_paged(upcast_f64(d.q), upcast_f64(d.k_pool), upcast_f64(d.v_pool),
                                  d.block_table.numpy(), d.seq_lens.numpy(), 16, d.scale,
                                  layout=d.layout)
        eo = float(np.abs(o1 - ro).max())
        el = float(np.abs(l1 - rl).max())
        say(f"  max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL and el <= TOL


def test_noalloc_decode_rejects_requests_beyond_the_scratch():
    say("noalloc decode: a request larger than the static scratch is rejected")
    d = decode_inputs(2, 32, 8, 128, seed=5, lmin=16, lmax=64, layout="rowmajor")
    # 2 sequences whose table rows hold 33000 blocks: 1032 splits each
    bt = torch.full((2, 33000), -1, dtype=torch.int32)
    bt[:, : d.block_table.shape[1]] = d.block_table
    need = A.attn_decode_workspace_bytes(2, 32, 128, 33000, 16)
    assert need > A.DECODE_STATIC_SCRATCH_BYTES
    with pytest.raises(A.AttnError) as e:
        A.decode_paged_noalloc(d.q.cuda(), d.k_pool.cuda(), d.v_pool.cuda(), bt.cuda(),
                               d.seq_lens.cuda(), 16, d.scale)
    assert e.value.status == -7
