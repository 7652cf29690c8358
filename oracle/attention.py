"""Plain fp64 attention, written from the definitions on the source pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Deliberately slow and
obvious: scores are materialised (in row blocks, to bound memory), masked,
soft-maxed and multiplied by V.  No tiling, fusion or reordering beyond what
the definitions state.  Inputs are numpy float64 arrays (the exact upcast of
the bf16/f32 tensors the GPU receives).

Sources (cited by page title and section):
  [FA]    "flash-attention与TensorRT-LLM集成：大语言模型推理优化",
          sections "背景与痛点分析" and "FlashAttention工作原理": FlashAttention
          is an *exact* attention computed IO-aware, so its result is the plain
          softmax(scale * Q K^T) V.
  [GQA]   "TensorRT对Grouped Query Attention的支持进展", sub-sections
          "技术演进背景" (query heads are split into groups; each group shares
          one K/V head) and "图优化与算子融合" (the repeat_kv plugin repeats
          each K/V head for the query heads of its group).
  [KV]    "LLM推理优化技术综述：KVCache、PageAttention、FlashAttention、MQA、GQA",
          parts on the autoregressive KV cache and PageAttention (a block table
          maps a sequence's contiguous logical blocks to non-contiguous
          physical blocks), and "TensorRT-LLM：大模型推理加速的工业级引擎",
          PagedAttention section.
  [BLASST] "高效部署稀疏注意力加速方案：BLASST方法详解与实践指南", section
          "架构与组件": a running maximum of the attention scores from the
          blockwise online softmax, a threshold lambda deciding whether a
          block matters, and skipping exp, the V load and the matmul for
          blocks that do not.

Readings where the pages are silent (each also listed in the design notes):
  * layout [B, H, S, D]; query head h reads K/V head h // (Hq // Hkv)
    (contiguous groups, the repeat_kv reading of [GQA]);
  * causal: key j visible to query i iff j <= i (equal query/key lengths);
  * LSE = natural log of sum_j exp(s_ij) over visible keys, s including scale;
  * decode: the single new query sees all L cached tokens (no mask);
  * block skip: whole T x T tiles per query head, ascending key-tile order,
    strict test (tile row max) - (running max) < ln(lambda), a tile skipped
    only when every one of its rows passes the test;
  * FP8 KV cache: E4M3 codes (the "FN" variant: no infinities, S.1111.111 is
    NaN) with one fp32 scale per pool, cached value = scale * code value.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = ["kv_head_of", "ref_prefill", "ref_decode_paged", "ref_blockskip", "pool_rows",
           "ref_decode_paged_blockskip", "ref_prefill_paged", "fp8_e4m3_value",
           "fp8_pool_rows", "ref_decode_paged_fp8"]


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """[GQA]: query heads form Hkv contiguous groups of Hq/Hkv heads; group g
    shares K/V head g (each K/V head repeated Hq/Hkv times in a row)."""
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def _softmax_rows(s: np.ndarray):
    """Row softmax of a score block whose masked entries are -inf.

    Returns (P, lse) with P = exp(s - lse) and lse = ln sum_j exp(s_ij);
    rows with no visible entry get P = 0 and lse = -inf.
    """
    m = np.max(s, axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe)
    z = np.sum(e, axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty, 0.0, e / np.where(z == 0, 1.0, z))
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(z == 0, 1.0, z)))
    return p, lse[:, 0]


def ref_prefill(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool,
                scale: float, rows: Optional[Sequence[int]] = None,
                row_block: int = 1024):
    """Exact attention [FA] with GQA head sharing [GQA].

    q: [B, Hq, S, D], k/v: [B, Hkv, S, D] float64.
    rows: optional query positions to evaluate (every (b, h) uses the same
    positions); default all S positions.
    Returns (O [B, Hq, R, D], LSE [B, Hq, R]) in float64.
    For each (b, h) with g = kv_head_of(h): s_ij = scale * <q_i, k_j>;
    keys with j > i are masked when causal; P = softmax over visible keys;
    O_i = sum_j P_ij v_j; LSE_i = ln sum_j exp(s_ij).
    """
    B, Hq, S, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    assert (Bk, Dk) == (B, D) and v.shape == k.shape
    assert Sk == S, "query and key lengths are equal in prefill"
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    out = np.zeros((B, Hq, R, D), dtype=np.float64)
    lse = np.zeros((B, Hq, R), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kg, vg = k[b, g], v[b, g]
            for r0 in range(0, R, row_block):
                ri = rows[r0:r0 + row_block]
                # causal: keys past the block's last row are masked for every
                # row of the block, so their scores are not formed
                nk = int(ri.max()) + 1 if causal else S
                s = scale * (q[b, h, ri, :] @ kg[:nk].T)        # [rb, nk]
                if causal:
                    s = np.where(np.arange(nk)[None, :] <= ri[:, None], s, -np.inf)
                p, l = _softmax_rows(s)
                out[b, h, r0:r0 + row_block] = p @ vg[:nk]
                lse[b, h, r0:r0 + row_block] = l
    return out, lse


def pool_rows(pool: np.ndarray, layout: str, which: str) -> np.ndarray:
    """View a K or V pool as [NB, Hkv, block_size, D] (token rows).

    "rowmajor" pools already are.  In the "mfma" layout each (block, head)
    run stores K as 8-element chunks, chunk-major ([D/8, block_size, 8]),
    and V transposed ([D, block_size]); only the order inside the run
    differs, so this is a pure index permutation."""
    if layout == "rowmajor":
        return pool
    if layout != "mfma":
        raise ValueError(layout)
    if which == "k":
        NB, Hkv, nc, bs, eight = pool.shape
        return pool.transpose(0, 1, 3, 2, 4).reshape(NB, Hkv, bs, nc * eight)
    return pool.transpose(0, 1, 3, 2)


def ref_decode_paged(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     block_table: np.ndarray, seq_lens: np.ndarray,
                     block_size: int, scale: float, layout: str = "rowmajor"):
    """Decode attention over a paged KV cache [KV].

    q: [N, Hq, D]; k_pool/v_pool: token rows [NB, Hkv, block_size, D] after
    :func:`pool_rows`; block_table: [N, max_blocks] (entry j = physical block
    holding logical block j); seq_lens: [N].  Cached token t of sequence n
    lives in physical block block_table[n, t // block_size], slot
    t % block_size.  The new query sees all L = seq_lens[n] cached tokens.
    Returns (O [N, Hq, D], LSE [N, Hq]); a sequence with L = 0 gets O = 0,
    LSE = -inf.
    """
    k_pool = pool_rows(k_pool, layout, "k")
    v_pool = pool_rows(v_pool, layout, "v")
    N, Hq, D = q.shape
    NB, Hkv, bs, Dk = k_pool.shape
    assert bs == block_size and Dk == D
    out = np.zeros((N, Hq, D), dtype=np.float64)
    lse = np.full((N, Hq), -np.inf, dtype=np.float64)
    for n in range(N):
        L = int(seq_lens[n])
        if L == 0:
            continue
        t = np.arange(L)
        phys = block_table[n, t // block_size].astype(np.int64)
        if np.any(phys < 0) or np.any(phys >= NB):
            raise ValueError(f"sequence {n}: block table entry out of range")
        slot = t % block_size
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kn = k_pool[phys, g, slot, :]                     # [L, D] logical order
            vn = v_pool[phys, g, slot, :]
            s = scale * (kn @ q[n, h])                         # [L]
            p, l = _softmax_rows(s[None, :])
            out[n, h] = p[0] @ vn
            lse[n, h] = l[0]
    return out, lse


def ref_blockskip(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, scale: float,
                  lam: float, tile: int, qtiles: Optional[Sequence[int]] = None):
    """Causal attention with BLASST block skipping [BLASST].

    The kernel walks key tiles kt = 0, 1, ..., qt in ascending order for each
    query tile qt (tile x tile blocks per query head) and keeps the running
    row maximum m of the scaled scores.  For tile kt it forms the tile row
    maxima tm_r (-inf where row r sees no key of the tile) and calls row r
    negligible iff tm_r = -inf, or m_r > -inf and tm_r - m_r < ln(lam).  The
    tile is skipped when all its rows are negligible: its exp, V load and P.V
    are left out.  Because a skipped tile has tm_r < m_r for every row (ln lam
    < 0), folding it into the maximum changes nothing, so the running max
    before tile kt equals the plain prefix maximum over ALL tiles kt' < kt;
    that is what is evaluated here (a cumulative maximum over the tile row
    maxima, shifted by one tile).  Keys of tiles past qt are masked for every
    row of query tile qt, so their scores are not formed.

    Returns (O [B,Hq,R,D], LSE [B,Hq,R], skip [B,Hq,nQ,nK] bool,
    gap [B,Hq,nQ,nK] float64) for the chosen query tiles (default: all),
    where R = rows of those tiles, skip[...,i,kt] refers to qtiles[i], and
    gap = max_r (tm_r - m_r) (+inf at kt = 0, -inf where kt > qt).
    """
    if not (0.0 < lam < 1.0):
        raise ValueError("lambda must lie in (0, 1)")
    B, Hq, S, D = q.shape
    _, Hkv, Sk, _ = k.shape
    assert Sk == S
    nT = (S + tile - 1) // tile
    qtiles = np.arange(nT) if qtiles is None else np.asarray(qtiles, dtype=np.int64)
    ln_lam = math.log(lam)
    row_list = [np.arange(qt * tile, min(S, (qt + 1) * tile)) for qt in qtiles]
    R = sum(len(r) for r in row_list)
    out = np.zeros((B, Hq, R, D))
    lse = np.zeros((B, Hq, R))
    skip = np.zeros((B, Hq, len(qtiles), nT), dtype=bool)
    gap = np.full((B, Hq, len(qtiles), nT), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kg, vg = k[b, g], v[b, g]
            r_out = 0
            for i, qt in enumerate(qtiles):
                ri = row_list[i]
                nt = int(qt) + 1                       # key tiles 0..qt
                nk = min(S, nt * tile)                 # their keys
                s = scale * (q[b, h, ri, :] @ kg[:nk].T)                # [R, nk]
                vis = np.arange(nk)[None, :] <= ri[:, None]
                s = np.where(vis, s, -np.inf)
                # tile row maxima tm[r, kt], kt = 0..qt (a partial last tile
                # is padded with -inf, which leaves its maxima unchanged)
                padded = np.full((len(ri), nt * tile), -np.inf)
                padded[:, :nk] = s
                tm = padded.reshape(len(ri), nt, tile).max(axis=2)      # [R, nt]
                # running maximum before tile kt: maximum over tiles 0..kt-1
                m_prev = np.concatenate([np.full((len(ri), 1), -np.inf),
                                         np.maximum.accumulate(tm, axis=1)[:, :-1]], axis=1)
                with np.errstate(invalid="ignore"):
                    d = tm - m_prev
                neg = np.isneginf(tm) | (np.isfinite(m_prev) & (d < ln_lam))
                skip[b, h, i, :nt] = np.all(neg, axis=0)
                gap[b, h, i, :nt] = np.max(d, axis=0)
                gap[b, h, i, 0] = np.inf
                keep = ~np.repeat(skip[b, h, i, :nt], tile)[:nk]
                s = np.where(keep[None, :], s, -np.inf)
                p, l = _softmax_rows(s)
                out[b, h, r_out:r_out + len(ri)] = p @ vg[:nk]
                lse[b, h, r_out:r_out + len(ri)] = l
                r_out += len(ri)
    return out, lse, skip, gap


def ref_decode_paged_blockskip(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                               block_table: np.ndarray, seq_lens: np.ndarray,
                               block_size: int, scale: float, *, lam: float,
                               split_tokens: int, layout: str = "rowmajor"):
    """Paged decode [KV] with BLASST block skipping [BLASST] inside each split.

    The cached tokens of sequence n are cut into splits of ``split_tokens``
    (a multiple of block_size) processed independently, as a split-KV
    decode does; inside a split the pool blocks are walked in ascending
    order.  For K/V head g and block b of a split, every query head h of the
    group has the block maximum tm_h (scaled scores of the block's cached
    tokens) and the running maximum m_h over the split's earlier blocks.  The
    block is skipped when, for every h, m_h > -inf and tm_h - m_h < ln(lam):
    its V load, exp and P.V are left out, for the whole group at once (the V
    block is shared).  The first block of a split is never skipped.  A
    skipped block has tm_h < m_h for every h, so folding it into the maximum
    changes nothing and m_h is the plain prefix maximum over the split's
    earlier blocks, which is what is evaluated here.

    Returns (O [N,Hq,D], LSE [N,Hq], skip [N,Hkv,max_blocks] bool,
    gap [N,Hkv,max_blocks]) with O/LSE the attention over the kept blocks'
    tokens, gap = max_h (tm_h - m_h) (+inf at a split's first block, -inf
    for unused blocks); skip <=> gap < ln(lam).
    """
    if not (0.0 < lam < 1.0):
        raise ValueError("lambda must lie in (0, 1)")
    if split_tokens % block_size:
        raise ValueError("split_tokens must be a multiple of block_size")
    k_pool = pool_rows(k_pool, layout, "k")
    v_pool = pool_rows(v_pool, layout, "v")
    N, Hq, D = q.shape
    NB, Hkv, bs, _ = k_pool.shape
    G = Hq // Hkv
    MB = block_table.shape[1]
    bps = split_tokens // block_size
    ln_lam = math.log(lam)
    out = np.zeros((N, Hq, D))
    lse = np.full((N, Hq), -np.inf)
    skip = np.zeros((N, Hkv, MB), dtype=bool)
    gap = np.full((N, Hkv, MB), -np.inf)
    for n in range(N):
        L = int(seq_lens[n])
        if L == 0:
            continue
        nb = (L + bs - 1) // bs
        phys = block_table[n, :nb].astype(np.int64)
        if np.any(phys < 0) or np.any(phys >= NB):
            raise ValueError(f"sequence {n}: block table entry out of range")
        t = np.arange(L)
        for g in range(Hkv):
            kn = k_pool[phys[t // bs], g, t % bs, :]           # [L, D]
            vn = v_pool[phys[t // bs], g, t % bs, :]
            s = scale * (q[n, g * G:(g + 1) * G] @ kn.T)       # [G, L]
            # block maxima [G, nb]
            tm = np.stack([s[:, b * bs:min(L, (b + 1) * bs)].max(axis=1) for b in range(nb)], 1)
            keep = np.ones(L, dtype=bool)
            for b in range(nb):
                first = b % bps == 0
                if first:
                    gap[n, g, b] = np.inf
                    continue
                m_prev = tm[:, (b // bps) * bps:b].max(axis=1)
                d = tm[:, b] - m_prev
                gap[n, g, b] = float(d.max())
                if np.all(d < ln_lam):
                    skip[n, g, b] = True
                    keep[b * bs:min(L, (b + 1) * bs)] = False
            sk = np.where(keep[None, :], s, -np.inf)
            p, l = _softmax_rows(sk)
            out[n, g * G:(g + 1) * G] = p @ vn
            lse[n, g * G:(g + 1) * G] = l
    return out, lse, skip, gap


def ref_prefill_paged(q: np.ndarray, cu_seqlens_q: np.ndarray, k_pool: np.ndarray,
                      v_pool: np.ndarray, block_table: np.ndarray, seq_lens_k: np.ndarray,
                      block_size: int, scale: float, layout: str = "rowmajor"):
    """Chunked / variable-length prefill over the paged KV cache [KV] (the
    prefill-with-KV-cache case of the FlashAttention integration page).

    Sequence n has Sk = seq_lens_k[n] tokens whose K/V are in the pool
    (gathered through its block-table row as in :func:`ref_decode_paged`);
    its Sq = cu_seqlens_q[n+1] - cu_seqlens_q[n] queries, rows
    cu_seqlens_q[n] .. of the packed q [total_q, Hq, D], are its LAST Sq
    positions: query i sits at position Sk - Sq + i and sees the keys
    j <= Sk - Sq + i (causal, bottom-right aligned).
    Returns (O [total_q, Hq, D], LSE [total_q, Hq]).
    """
    k_pool = pool_rows(k_pool, layout, "k")
    v_pool = pool_rows(v_pool, layout, "v")
    total_q, Hq, D = q.shape
    NB, Hkv, bs, _ = k_pool.shape
    N = len(seq_lens_k)
    out = np.zeros((total_q, Hq, D))
    lse = np.zeros((total_q, Hq))
    for n in range(N):
        r0, r1 = int(cu_seqlens_q[n]), int(cu_seqlens_q[n + 1])
        Sq, Sk = r1 - r0, int(seq_lens_k[n])
        if Sq == 0:
            continue
        if Sq > Sk:
            raise ValueError(f"sequence {n}: more queries than cached tokens")
        t = np.arange(Sk)
        phys = block_table[n, t // bs].astype(np.int64)
        if np.any(phys < 0) or np.any(phys >= NB):
            raise ValueError(f"sequence {n}: block table entry out of range")
        pos = Sk - Sq + np.arange(Sq)
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            kn = k_pool[phys, g, t % bs, :]
            vn = v_pool[phys, g, t % bs, :]
            s = scale * (q[r0:r1, h, :] @ kn.T)                     # [Sq, Sk]
            s = np.where(t[None, :] <= pos[:, None], s, -np.inf)
            p, l = _softmax_rows(s)
            out[r0:r1, h] = p @ vn
            lse[r0:r1, h] = l
    return out, lse


def fp8_e4m3_value(code) -> np.ndarray:
    """fp64 value of FP8 E4M3 codes.

    FP8 with the E4M3 encoding is one of the low-precision formats the
    TensorRT-LLM page lists ("TensorRT-LLM：大模型推理加速的工业级引擎",
    六大核心优化技术 / 量化, and the 深入版解读 note on E4M3/E5M2).  The page
    does not spell the encoding out; this is the common E4M3 "FN" format:
    bit 7 sign, bits 6..3 exponent e with bias 7, bits 2..0 mantissa m.
      e = 0:                  (-1)^s * (m / 8) * 2^(1 - 7)   (subnormal)
      0 < e, not (e = 15 and m = 7): (-1)^s * (1 + m / 8) * 2^(e - 7)
      e = 15 and m = 7:       NaN (there are no infinities; largest finite 448)
    """
    c = np.asarray(code).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** (1 - 7), (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


def fp8_pool_rows(pool: np.ndarray, which: str, D: int, block_size: int = 16) -> np.ndarray:
    """Token rows [NB, Hkv, block_size, D] of an FP8 pool in the MFMA-native
    byte order (one contiguous run of block_size * D bytes per (block, head)).

    Inside a run, with c = d // 16:
      K byte (t, d) at (c // 4) * 1024 + ((c % 4) * 16 + t) * 16 + d % 16
      V byte (t, d) at (b // 4) * 1024 + ((t // 4) * 16 + d % 16) * 16
                       + (b % 4) * 4 + t % 4,    b = d // 16
    (block_size = 16).  Returns the codes rearranged; a pure permutation."""
    if block_size != 16 or D % 64:
        raise ValueError("the FP8 pool layout needs block_size 16 and D % 64 == 0")
    NB, Hkv = pool.shape[:2]
    run = pool.reshape(NB, Hkv, block_size * D)
    t = np.arange(block_size)[:, None]
    d = np.arange(D)[None, :]
    c = d // 16
    if which == "k":
        off = (c // 4) * 1024 + ((c % 4) * 16 + t) * 16 + d % 16
    elif which == "v":
        off = (c // 4) * 1024 + ((t // 4) * 16 + d % 16) * 16 + (c % 4) * 4 + t % 4
    else:
        raise ValueError(which)
    return run[:, :, off]


def ref_decode_paged_fp8(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                         block_table: np.ndarray, seq_lens: np.ndarray, block_size: int,
                         scale: float, k_scale: float, v_scale: float):
    """Decode attention over an FP8 paged KV cache [KV]: the codes are
    decoded (:func:`fp8_e4m3_value`), multiplied by their pool's scale, and
    the plain decode of :func:`ref_decode_paged` runs on those values.
    k_pool / v_pool: uint8 codes [NB, Hkv, block_size * D] in the byte order
    of :func:`fp8_pool_rows`."""
    D = q.shape[-1]
    k = k_scale * fp8_e4m3_value(fp8_pool_rows(k_pool, "k", D, block_size))
    v = v_scale * fp8_e4m3_value(fp8_pool_rows(v_pool, "v", D, block_size))
    return ref_decode_paged(q, k, v, block_table, seq_lens, block_size, scale)
