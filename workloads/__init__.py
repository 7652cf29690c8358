"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out in memory.  It holds
none of the attention arithmetic, so both the fp64 oracle and the HIP library
can be fed from it without sharing any of the method's code.

Every tensor is produced on the host (CPU).  Floating-point samples are drawn
as float32 from numpy's PCG64 generator and then rounded to the working dtype
with a round-to-nearest-even cast (torch's ``Tensor.to(torch.bfloat16)``).
Consumers must treat the rounded tensor as THE input: the oracle upcasts it
exactly to fp64, the GPU reads it as is.

Shapes follow the prefill problem statement on the FlashAttention/TensorRT-LLM
page ("flash-attention与TensorRT-LLM集成", section on how FlashAttention
works: Q, K, V are split into blocks), with the grouped-query head layout of
the TensorRT GQA page ("TensorRT对Grouped Query Attention的支持进展",
technical background: query heads split into groups that share one K/V head)
and the paged KV cache of the PagedAttention description ("TensorRT-LLM：大模型
推理加速的工业级引擎", PagedAttention section: fixed-size blocks plus a block
table mapping logical to physical blocks).

Layouts:
  * prefill Q/O: [B, Hq, S, D]; K/V: [B, Hkv, S, D] (contiguous, row-major)
  * decode q/o: [N, Hq, D]; block_table: int32 [N, max_blocks_per_seq]
    (padding -1); seq_lens: int32 [N]; pools in one of two layouts, both with
    one contiguous (block, head) run of block_size * D elements:
      "rowmajor": k_pool, v_pool [NB, Hkv, block_size, D]
      "mfma":     k_pool [NB, Hkv, D/8, block_size, 8]  (8-element chunks, chunk-major)
                  v_pool [NB, Hkv, D, block_size]       (V transposed within the block)
    FP8 pools (E4M3 codes, one byte each, block_size 16, D % 64 == 0) have one
    byte order, again one contiguous run of 16 * D bytes per (block, head):
      k_pool [NB, Hkv, D/64, 4, 16 tokens, 16]  dims (4i + g) * 16 + w at [i, g, t, w]
      v_pool [NB, Hkv, D/64, 4, 16, 4, 4]       token 4j + u, dim (4i + b) * 16 + r
                                                 at [i, j, r, b, u]
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = [
    "PrefillInputs", "DecodeInputs", "CONFIGS",
    "prefill_inputs", "blockskip_inputs", "decode_inputs", "shared_prefix_decode_inputs",
    "unshared_copy", "paged_prefill_inputs", "PagedPrefillInputs", "to_dtype",
    "upcast_f64", "prefill_flops", "Fp8DecodeInputs", "fp8_decode_inputs",
]


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a float32 numpy array to ``dtype`` ("bf16" or "f32") on the CPU."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(f"unknown dtype {dtype!r}")


def upcast_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a CPU bf16/f32 tensor to a float64 numpy array."""
    return t.to(torch.float64).numpy()


def prefill_flops(B: int, Hq: int, S: int, D: int, causal: bool) -> int:
    """Algorithmic flops of one prefill: 2*D per visible (query, key) pair for
    Q.K^T and 2*D for P.V.  Causal visible pairs per head: S(S+1)/2."""
    pairs = S * (S + 1) // 2 if causal else S * S
    return 4 * B * Hq * D * pairs


@dataclasses.dataclass
class PrefillInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    causal: bool
    scale: float
    dtype: str
    seed: int
    # block-skip structure (None for plain prefill workloads)
    sink_rows: Optional[np.ndarray] = None
    boosted_rows: Optional[np.ndarray] = None
    boost_dim: Optional[int] = None


@dataclasses.dataclass
class DecodeInputs:
    q: torch.Tensor            # [N, Hq, D]
    k_pool: torch.Tensor       # [NB, Hkv, block_size, D]
    v_pool: torch.Tensor       # [NB, Hkv, block_size, D]
    block_table: torch.Tensor  # int32 [N, max_blocks]
    seq_lens: torch.Tensor     # int32 [N]
    block_size: int
    N: int
    Hq: int
    Hkv: int
    D: int
    max_blocks: int
    scale: float
    dtype: str
    seed: int
    perm: np.ndarray           # logical block id -> physical block id
    layout: str = "rowmajor"

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    def kv_bytes(self) -> int:
        """Bytes of K and V the decode must read: sum_n L_n * Hkv * D * 2 tensors."""
        esize = 2 if self.dtype == "bf16" else 4
        return int(self.seq_lens.to(torch.int64).sum()) * self.Hkv * self.D * 2 * esize


def prefill_inputs(B: int, Hq: int, Hkv: int, S: int, D: int, *, seed: int,
                   dtype: str = "bf16", causal: bool = True,
                   scale: Optional[float] = None) -> PrefillInputs:
    """i.i.d. N(0,1) Q, K, V drawn in that order as whole [B,H,S,D] tensors."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return PrefillInputs(to_dtype(q, dtype), to_dtype(k, dtype), to_dtype(v, dtype),
                         B, Hq, Hkv, S, D, causal, float(scale), dtype, seed)


def blockskip_inputs(B: int, Hq: int, Hkv: int, S: int, D: int, *, seed: int,
                     amplitude: float = 3.0, n_sinks: int = 64,
                     boosted: str = "random_half", dtype: str = "bf16",
                     scale: Optional[float] = None) -> PrefillInputs:
    """Attention-sink structure for the block-skip workload.

    Q, K, V are N(0,1) as in :func:`prefill_inputs`.  Then one coordinate
    ``k`` in [0, D) is drawn (u = e_k), ``n_sinks`` key positions are drawn
    without replacement (shared by every KV head and batch) and get
    ``amplitude * e_k`` added, and half of the query positions get
    ``amplitude * u`` added (shared by every query head and batch).
    ``boosted`` is "random_half" (S/2 positions drawn without replacement) or
    "second_half" (positions S/2 .. S-1, the stress variant).  The boost is
    added to the float32 sample before rounding to ``dtype``.

    ``boosted="split_tiles"`` builds tiles whose two 32-row halves disagree:
    key 0 is the only sink and every query row is boosted along u, and a
    second coordinate k2 != k (w = e_k2, drawn after k) gets ``amplitude *
    w`` on key 64t + 17 of every 64-key tile t and on the query rows r with
    r % 64 >= 32.  Rows of the first half of each 64-row block then find
    every key tile after the first negligible against key 0, while rows of
    the second half do not (``n_sinks`` is ignored).
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, S, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, D), dtype=np.float32)
    kdim = int(rng.integers(0, D))
    if boosted == "split_tiles":
        kdim2 = (kdim + 1 + int(rng.integers(0, D - 1))) % D
        sinks = np.array([0])
        spots = np.arange(17, S, 64)
        rows = np.arange(S)
        k[:, :, sinks, kdim] += np.float32(amplitude)
        q[:, :, :, kdim] += np.float32(amplitude)
        k[:, :, spots, kdim2] += np.float32(amplitude)
        q[:, :, rows[rows % 64 >= 32], kdim2] += np.float32(amplitude)
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        return PrefillInputs(to_dtype(q, dtype), to_dtype(k, dtype), to_dtype(v, dtype),
                             B, Hq, Hkv, S, D, True, float(scale), dtype, seed,
                             sink_rows=sinks, boosted_rows=rows, boost_dim=kdim)
    sinks = np.sort(rng.choice(S, size=min(n_sinks, S), replace=False))
    if boosted == "random_half":
        rows = np.sort(rng.choice(S, size=S // 2, replace=False))
    elif boosted == "second_half":
        rows = np.arange(S // 2, S)
    else:
        raise ValueError(boosted)
    k[:, :, sinks, kdim] += np.float32(amplitude)
    q[:, :, rows, kdim] += np.float32(amplitude)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return PrefillInputs(to_dtype(q, dtype), to_dtype(k, dtype), to_dtype(v, dtype),
                         B, Hq, Hkv, S, D, True, float(scale), dtype, seed,
                         sink_rows=sinks, boosted_rows=rows, boost_dim=kdim)


def decode_inputs(N: int, Hq: int, Hkv: int, D: int, *, seed: int,
                  lmin: int = 512, lmax: int = 4096, block_size: int = 16,
                  tail: str = "zero", dtype: str = "bf16",
                  lens: Optional[list] = None,
                  scale: Optional[float] = None, layout: str = "rowmajor",
                  sink_amplitude: float = 0.0, sink_frac: float = 0.0) -> DecodeInputs:
    """Paged KV-cache decode inputs.

    Draw order: the N context lengths (uniform integers on [lmin, lmax],
    inclusive) unless ``lens`` is given, then q [N,Hq,D], then for each
    sequence its logical K and V ([L,Hkv,D] each, K first), then one random
    permutation of the NB = sum ceil(L/block_size) physical blocks.  Logical
    block j of sequence n (numbered sequence-major, ``base_n + j``) lives in
    physical block ``perm[base_n + j]``.  Unused slots of each sequence's last
    block hold zeros (``tail="zero"``) or NaN (``tail="nan"``, which a correct
    kernel never reads).  Padding entries of the block table are -1.
    ``layout`` only rearranges elements inside each (block, head) run (see
    the module docstring); the random draws are identical for both.

    With ``sink_amplitude`` > 0 (a labelled stress input for block skipping)
    three more draws follow the permutation: one dimension kd, then for
    each sequence a uniform draw per cached token; token 0 and the tokens
    whose draw is below ``sink_frac`` are sinks.  The amplitude is added to
    q[:, :, kd] and to K[sink, :, kd] before the dtype rounding, so sinks
    dominate the scores of every query head.
    """
    rng = np.random.default_rng(seed)
    if lens is None:
        lens_np = rng.integers(lmin, lmax, size=N, endpoint=True).astype(np.int64)
    else:
        lens_np = np.asarray(lens, dtype=np.int64)
        assert lens_np.shape == (N,)
    q = rng.standard_normal((N, Hq, D), dtype=np.float32)
    nblk = [(int(L) + block_size - 1) // block_size for L in lens_np]
    NB = int(sum(nblk))
    max_blocks = max(1, max(nblk) if nblk else 1)
    fill = np.nan if tail == "nan" else 0.0
    kp = np.full((NB, Hkv, block_size, D), fill, dtype=np.float32)
    vp = np.full((NB, Hkv, block_size, D), fill, dtype=np.float32)
    logical_k, logical_v = [], []
    for n in range(N):
        L = int(lens_np[n])
        logical_k.append(rng.standard_normal((L, Hkv, D), dtype=np.float32))
        logical_v.append(rng.standard_normal((L, Hkv, D), dtype=np.float32))
    perm = rng.permutation(NB) if NB > 0 else np.zeros(0, dtype=np.int64)
    if sink_amplitude:
        kd = int(rng.integers(D))
        q[:, :, kd] += np.float32(sink_amplitude)
        for n in range(N):
            u = rng.random(int(lens_np[n]))
            sink = u < sink_frac
            if len(sink):
                sink[0] = True
            logical_k[n][sink, :, kd] += np.float32(sink_amplitude)
    table = np.full((N, max_blocks), -1, dtype=np.int32)
    base = 0
    for n in range(N):
        L = int(lens_np[n])
        for j in range(nblk[n]):
            p = int(perm[base + j])
            table[n, j] = p
            t0, t1 = j * block_size, min(L, (j + 1) * block_size)
            # [tokens, Hkv, D] -> [Hkv, tokens, D]
            kp[p, :, : t1 - t0, :] = logical_k[n][t0:t1].transpose(1, 0, 2)
            vp[p, :, : t1 - t0, :] = logical_v[n][t0:t1].transpose(1, 0, 2)
        base += nblk[n]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kp, vp = _to_layout(kp, vp, layout, block_size, D)
    return DecodeInputs(
        q=to_dtype(q, dtype), k_pool=to_dtype(kp, dtype), v_pool=to_dtype(vp, dtype),
        block_table=torch.from_numpy(table), seq_lens=torch.from_numpy(lens_np.astype(np.int32)),
        block_size=block_size, N=N, Hq=Hq, Hkv=Hkv, D=D, max_blocks=max_blocks,
        scale=float(scale), dtype=dtype, seed=seed, perm=perm, layout=layout)


def shared_prefix_decode_inputs(n_prompts: int, n_samples: int, Hq: int, Hkv: int, D: int, *,
                                seed: int, prefix_len: int, suffix_min: int, suffix_max: int,
                                block_size: int = 16, tail: str = "zero", dtype: str = "bf16",
                                scale: Optional[float] = None, layout: str = "rowmajor"):
    """Decode inputs whose sequences share prompt blocks (copy-on-write).

    Per the PageAttention part of the "LLM推理优化技术综述" page, several
    outputs generated from one prompt share the prompt's K/V blocks, and a
    block is copied only when it is written to.  Sequence n = p * n_samples
    + m (sample m of prompt p) holds the prompt's prefix_len tokens followed
    by its own suffix.  The prompt's full blocks (prefix_len // block_size of
    them) are physical blocks referenced by all its samples' table rows; the
    partly filled last prompt block is copied into each sample, which then
    appends its own tokens there.

    Draw order: the N suffix lengths (uniform integers on [suffix_min,
    suffix_max]), q [N,Hq,D], per prompt its prefix K then V
    ([prefix_len,Hkv,D]), per sequence its suffix K then V, then one
    permutation of the physical blocks (shared blocks numbered first, prompt
    by prompt, then each sequence's private blocks).

    Returns (DecodeInputs, logical) where logical[n] = (K, V) float32 arrays
    [L, Hkv, D] of sequence n before the dtype rounding.
    """
    rng = np.random.default_rng(seed)
    bs = block_size
    N = n_prompts * n_samples
    suffix = rng.integers(suffix_min, suffix_max, size=N, endpoint=True).astype(np.int64)
    lens = prefix_len + suffix
    q = rng.standard_normal((N, Hq, D), dtype=np.float32)
    pre = []
    for _ in range(n_prompts):
        pk = rng.standard_normal((prefix_len, Hkv, D), dtype=np.float32)
        pv = rng.standard_normal((prefix_len, Hkv, D), dtype=np.float32)
        pre.append((pk, pv))
    logical = []
    for n in range(N):
        sk = rng.standard_normal((int(suffix[n]), Hkv, D), dtype=np.float32)
        sv = rng.standard_normal((int(suffix[n]), Hkv, D), dtype=np.float32)
        pk, pv = pre[n // n_samples]
        logical.append((np.concatenate([pk, sk]), np.concatenate([pv, sv])))
    n_shared = prefix_len // bs
    nblk = [(int(L) + bs - 1) // bs for L in lens]
    NB = n_prompts * n_shared + sum(nb - n_shared for nb in nblk)
    max_blocks = max(nblk)
    perm = rng.permutation(NB)
    fill = np.nan if tail == "nan" else 0.0
    kp = np.full((NB, Hkv, bs, D), fill, dtype=np.float32)
    vp = np.full((NB, Hkv, bs, D), fill, dtype=np.float32)
    table = np.full((N, max_blocks), -1, dtype=np.int32)

    def put(phys, K, V, t0, t1):
        kp[phys, :, : t1 - t0, :] = K[t0:t1].transpose(1, 0, 2)
        vp[phys, :, : t1 - t0, :] = V[t0:t1].transpose(1, 0, 2)

    for p in range(n_prompts):
        for j in range(n_shared):
            phys = int(perm[p * n_shared + j])
            put(phys, pre[p][0], pre[p][1], j * bs, (j + 1) * bs)
            for m in range(n_samples):
                table[p * n_samples + m, j] = phys
    nxt = n_prompts * n_shared
    for n in range(N):
        K, V = logical[n]
        L = int(lens[n])
        for j in range(n_shared, nblk[n]):
            phys = int(perm[nxt])
            nxt += 1
            put(phys, K, V, j * bs, min(L, (j + 1) * bs))
            table[n, j] = phys
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kp, vp = _to_layout(kp, vp, layout, bs, D)
    d = DecodeInputs(
        q=to_dtype(q, dtype), k_pool=to_dtype(kp, dtype), v_pool=to_dtype(vp, dtype),
        block_table=torch.from_numpy(table), seq_lens=torch.from_numpy(lens.astype(np.int32)),
        block_size=bs, N=N, Hq=Hq, Hkv=Hkv, D=D, max_blocks=max_blocks,
        scale=float(scale), dtype=dtype, seed=seed, perm=perm, layout=layout)
    return d, logical


@dataclasses.dataclass
class PagedPrefillInputs:
    q: torch.Tensor             # [total_q, Hq, D] packed queries
    cu_seqlens_q: torch.Tensor  # int32 [N + 1]
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_table: torch.Tensor   # int32 [N, max_blocks]
    seq_lens_k: torch.Tensor    # int32 [N]
    block_size: int
    N: int
    Hq: int
    Hkv: int
    D: int
    max_blocks: int
    max_seqlen_q: int
    scale: float
    dtype: str
    layout: str

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])


def paged_prefill_inputs(ctx_lens: list, q_lens: list, Hq: int, Hkv: int, D: int, *, seed: int,
                         block_size: int = 16, tail: str = "zero", dtype: str = "bf16",
                         scale: Optional[float] = None,
                         layout: str = "rowmajor") -> PagedPrefillInputs:
    """Chunked prefill over a paged cache: sequence n has ctx_lens[n] earlier
    tokens and a new chunk of q_lens[n] tokens, all Sk = ctx + q of them in
    the pool.  Draw order: the packed queries [total_q, Hq, D], then per
    sequence its K then V ([Sk, Hkv, D]), then one permutation of the
    physical blocks (logical blocks numbered sequence-major)."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    ql = np.asarray(q_lens, dtype=np.int64)
    N = len(ctx)
    sk = ctx + ql
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    q = rng.standard_normal((int(cu[-1]), Hq, D), dtype=np.float32)
    nblk = [(int(L) + block_size - 1) // block_size for L in sk]
    NB = max(1, int(sum(nblk)))
    max_blocks = max(1, max(nblk))
    fill = np.nan if tail == "nan" else 0.0
    kp = np.full((NB, Hkv, block_size, D), fill, dtype=np.float32)
    vp = np.full((NB, Hkv, block_size, D), fill, dtype=np.float32)
    logical = []
    for n in range(N):
        L = int(sk[n])
        logical.append((rng.standard_normal((L, Hkv, D), dtype=np.float32),
                        rng.standard_normal((L, Hkv, D), dtype=np.float32)))
    perm = rng.permutation(NB)
    table = np.full((N, max_blocks), -1, dtype=np.int32)
    base = 0
    for n in range(N):
        L = int(sk[n])
        for j in range(nblk[n]):
            p = int(perm[base + j])
            table[n, j] = p
            t0, t1 = j * block_size, min(L, (j + 1) * block_size)
            kp[p, :, : t1 - t0, :] = logical[n][0][t0:t1].transpose(1, 0, 2)
            vp[p, :, : t1 - t0, :] = logical[n][1][t0:t1].transpose(1, 0, 2)
        base += nblk[n]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kp, vp = _to_layout(kp, vp, layout, block_size, D)
    return PagedPrefillInputs(
        q=to_dtype(q, dtype), cu_seqlens_q=torch.from_numpy(cu), k_pool=to_dtype(kp, dtype),
        v_pool=to_dtype(vp, dtype), block_table=torch.from_numpy(table),
        seq_lens_k=torch.from_numpy(sk.astype(np.int32)), block_size=block_size, N=N, Hq=Hq,
        Hkv=Hkv, D=D, max_blocks=max_blocks, max_seqlen_q=int(ql.max()) if N else 0,
        scale=float(scale), dtype=dtype, layout=layout)


def unshared_copy(d: DecodeInputs) -> DecodeInputs:
    """The same cache with every table entry pointing at a private copy of
    its block (data movement only: blocks are copied whole, in order)."""
    table = d.block_table.numpy()
    N, MB = table.shape
    used = [(n, j) for n in range(N) for j in range(MB) if table[n, j] >= 0]
    src = torch.tensor([int(table[n, j]) for n, j in used], dtype=torch.long)
    new_table = np.full_like(table, -1)
    for i, (n, j) in enumerate(used):
        new_table[n, j] = i
    return dataclasses.replace(d, k_pool=d.k_pool[src].clone(), v_pool=d.v_pool[src].clone(),
                               block_table=torch.from_numpy(new_table),
                               perm=np.arange(len(used)))


@dataclasses.dataclass
class Fp8DecodeInputs:
    """An FP8 copy of a bf16 decode problem: the K and V pools quantized to
    E4M3 codes with one scale per pool (code = round(x / scale), saturated to
    +-448; NaN tail slots stay NaN codes)."""
    base: DecodeInputs          # the bf16 problem (row-major pools); q, table, lengths
    k_pool: torch.Tensor        # uint8 [NB, Hkv, 16 * D], FP8 byte order
    v_pool: torch.Tensor
    k_scale: float
    v_scale: float
    k_codes: torch.Tensor       # uint8 [NB, Hkv, 16, D], the same codes as token rows
    v_codes: torch.Tensor
    k_rows: torch.Tensor        # float64 [NB, Hkv, 16, D] = scale * code value (torch's decoding)
    v_rows: torch.Tensor

    def kv_bytes(self) -> int:
        """Bytes of K and V the decode must read: sum_n L_n * Hkv * D * 2 tensors * 1 byte."""
        b = self.base
        return int(b.seq_lens.to(torch.int64).sum()) * b.Hkv * b.D * 2


def _fp8_quantize(pool: torch.Tensor):
    x = pool.to(torch.float32)
    finite = x[torch.isfinite(x)]
    amax = float(finite.abs().max()) if finite.numel() else 1.0
    scale = float(np.float32(max(amax, 1e-30) / 448.0))
    codes = (x / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    rows = codes.to(torch.float64) * scale
    return codes.view(torch.uint8), scale, rows


def _fp8_byte_order(codes: torch.Tensor, which: str) -> torch.Tensor:
    NB, Hkv, bs, D = codes.shape
    if which == "k":   # [NB, Hkv, t, i, g, w] -> [NB, Hkv, i, g, t, w]
        x = codes.reshape(NB, Hkv, bs, D // 64, 4, 16).permute(0, 1, 3, 4, 2, 5)
    else:              # [NB, Hkv, j, u, i, b, r] -> [NB, Hkv, i, j, r, b, u]
        x = codes.reshape(NB, Hkv, 4, 4, D // 64, 4, 16).permute(0, 1, 4, 2, 6, 5, 3)
    return x.contiguous().reshape(NB, Hkv, bs * D)


def fp8_decode_inputs(N: int, Hq: int, Hkv: int, D: int, *, seed: int,
                      **kw) -> Fp8DecodeInputs:
    """The decode problem of :func:`decode_inputs` (same draws; bf16 q,
    row-major pools) with its K and V pools quantized to FP8 E4M3.  Each
    pool gets scale = max|x| / 448 over its finite entries (as float32), and
    codes round(x / scale) (round to nearest even, torch's float8_e4m3fn
    conversion) in the FP8 byte order of the module docstring."""
    if D % 64:
        raise ValueError("FP8 pools need D % 64 == 0")
    kw.pop("layout", None)
    kw.pop("dtype", None)
    d = decode_inputs(N, Hq, Hkv, D, seed=seed, layout="rowmajor", dtype="bf16", **kw)
    if d.block_size != 16:
        raise ValueError("FP8 pools need block_size 16")
    kc, ks, kr = _fp8_quantize(d.k_pool)
    vc, vs, vr = _fp8_quantize(d.v_pool)
    return Fp8DecodeInputs(base=d, k_pool=_fp8_byte_order(kc, "k"), v_pool=_fp8_byte_order(vc, "v"),
                           k_scale=ks, v_scale=vs, k_codes=kc, v_codes=vc, k_rows=kr, v_rows=vr)


def _to_layout(kp: np.ndarray, vp: np.ndarray, layout: str, bs: int, D: int):
    """Rearrange row-major pools [NB, Hkv, bs, D] into ``layout``."""
    if layout == "mfma":
        if D % 8:
            raise ValueError("the mfma layout needs D % 8 == 0")
        NB, Hkv = kp.shape[:2]
        kp = np.ascontiguousarray(kp.reshape(NB, Hkv, bs, D // 8, 8).transpose(0, 1, 3, 2, 4))
        vp = np.ascontiguousarray(vp.transpose(0, 1, 3, 2))
    elif layout != "rowmajor":
        raise ValueError(layout)
    return kp, vp


# The five named workloads.  Sizes are the problem statement's; seeds are fixed
# so that every consumer (tests, bench, oracle timing) sees the same tensors.
CONFIGS = {
    "tiny_gqa_f32": dict(kind="prefill", B=1, Hq=4, Hkv=2, S=128, D=64, dtype="f32",
                         causal=True, seed=1001),
    "mha_causal_s2048": dict(kind="prefill", B=4, Hq=32, Hkv=32, S=2048, D=128, dtype="bf16",
                             causal=True, seed=1002),
    "gqa_causal_s8192": dict(kind="prefill", B=1, Hq=32, Hkv=8, S=8192, D=128, dtype="bf16",
                             causal=True, seed=1003),
    "paged_decode_gqa": dict(kind="decode", N=64, Hq=32, Hkv=8, D=128, lmin=512, lmax=4096,
                             block_size=16, dtype="bf16", seed=1004),
    "blockskip_s32768": dict(kind="blockskip", B=1, Hq=32, Hkv=8, S=32768, D=128, dtype="bf16",
                             amplitude=3.0, boosted="random_half", seed=1005,
                             lam=1e-3, tile=64),
}
