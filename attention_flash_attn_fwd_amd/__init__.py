"""Python binding of libattn.so (exact IO-aware attention for MI355X / gfx950).

Argument marshalling only: tensors are turned into device pointers and sizes,
the current HIP stream is passed along, and every computation runs in the HIP
kernels of libattn.so.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

The functions named like the C entry points (``attn_prefill``,
``attn_prefill_f32``, ``attn_prefill_blockskip``, ``attn_decode_paged``,
``attn_decode_workspace_bytes``, ``attn_status_string``, ...) take caller-allocated
torch tensors; ``prefill``, ``prefill_blockskip`` and ``decode_paged``
allocate the outputs and return them.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "AttnError", "lib_path", "load", "attn_status_string", "attn_arch_supported",
    "attn_prefill", "attn_prefill_f32", "attn_prefill_blockskip",
    "attn_decode_workspace_bytes", "attn_decode_paged", "attn_decode_paged_blockskip",
    "attn_prefill_paged", "attn_decode_paged_fp8", "attn_decode_paged_noalloc",
    "DECODE_STATIC_SCRATCH_BYTES",
    "prefill", "prefill_blockskip", "decode_paged", "decode_paged_blockskip", "prefill_paged",
    "decode_paged_fp8", "decode_paged_noalloc",
]

# ATTN_DECODE_STATIC_SCRATCH_BYTES of include/attn.h
DECODE_STATIC_SCRATCH_BYTES = 16 << 20

_LIB: Optional[ctypes.CDLL] = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float


class AttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {attn_status_string(status)} (status {status})")
        self.status = status


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")


def load() -> ctypes.CDLL:
    """Load libattn.so (built by attention_flash_attn_fwd_amd._build)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m attention_flash_attn_fwd_amd._build`")
    lib = ctypes.CDLL(path)
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [_I]
    lib.attn_arch_supported.restype = _I
    lib.attn_arch_supported.argtypes = [ctypes.c_char_p]
    pre = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]
    for name in ("attn_prefill", "attn_prefill_f32"):
        getattr(lib, name).restype = _I
        getattr(lib, name).argtypes = pre
    lib.attn_prefill_blockskip.restype = _I
    lib.attn_prefill_blockskip.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _I,
                                           _P, _P, _P]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
    lib.attn_decode_paged.restype = _I
    lib.attn_decode_paged.argtypes = [_P, _P, _P, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _I, _I,
                                      _F, _P, ctypes.c_size_t, _P]
    lib.attn_prefill_paged.restype = _I
    lib.attn_prefill_paged.argtypes = [_P, _P, _I, _I, _P, _P, _P, _P, _I, _I, _P, _P, _I, _I, _I,
                                       _I, _I, _I, _F, _P]
    lib.attn_decode_paged_noalloc.restype = _I
    lib.attn_decode_paged_noalloc.argtypes = [_P, _P, _P, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I,
                                              _I, _I, _F, _P]
    lib.attn_decode_paged_blockskip.restype = _I
    lib.attn_decode_paged_blockskip.argtypes = [_P, _P, _P, _P, _P, _I, _I, _P, _P, _I, _I, _I,
                                                _I, _I, _I, _F, _F, _P, _P, _P, ctypes.c_size_t,
                                                _P]
    lib.attn_decode_paged_fp8.restype = _I
    lib.attn_decode_paged_fp8.argtypes = [_P, _P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I,
                                          _F, _F, _F, _P, ctypes.c_size_t, _P]
    _LIB = lib
    return lib


def attn_status_string(status: int) -> str:
    return load().attn_status_string(int(status)).decode()


def attn_arch_supported(name: str) -> bool:
    return bool(load().attn_arch_supported(name.encode()))


# ------------------------------------------------------------------ helpers

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(st: int, where: str) -> None:
    if st != 0:
        raise AttnError(st, where)


def _dev(*ts):
    """All given tensors on one GPU, the current one: the library launches on
    the current device's stream and checks that device's architecture."""
    idx = None
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("tensors must live on the GPU")
        i = t.device.index if t.device.index is not None else torch.cuda.current_device()
        if idx is None:
            idx = i
        elif i != idx:
            raise ValueError("tensors must live on one GPU")
    if idx is not None and idx != torch.cuda.current_device():
        raise ValueError(f"tensors live on cuda:{idx} but the current device is "
                         f"cuda:{torch.cuda.current_device()}; call under torch.cuda.device({idx})")


# ---------------------------------------------------- C-ABI mirrors (in-place)

def attn_prefill(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """bf16 prefill into caller-allocated o [B,Hq,S,D] and lse [B,Hq,S] (or None)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _dev(q, k, v, o, lse)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16 \
            or o.dtype != torch.bfloat16:
        raise TypeError("attn_prefill takes bfloat16 tensors")
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (B, Hq, S)):
        raise ValueError("lse must be float32 [B,Hq,S]")
    st = load().attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, S, D,
                             int(bool(causal)), float(scale), _stream(stream))
    _check(st, "attn_prefill")


def attn_prefill_f32(q, k, v, o, lse, causal: bool, scale: float, stream=None) -> None:
    """float32 prefill into caller-allocated o and lse (or None)."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _dev(q, k, v, o, lse)
    for t in (q, k, v, o):
        if t.dtype != torch.float32:
            raise TypeError("attn_prefill_f32 takes float32 tensors")
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (B, Hq, S)):
        raise ValueError("lse must be float32 [B,Hq,S]")
    st = load().attn_prefill_f32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, S,
                                 D, int(bool(causal)), float(scale), _stream(stream))
    _check(st, "attn_prefill_f32")


def attn_prefill_blockskip(q, k, v, o, lse, scale: float, lam: float, tile: int = 64,
                           skip_bitmap=None, skipped_tiles=None, stream=None) -> None:
    """Causal bf16 prefill with block skipping; skipped_tiles (uint64/int64
    device scalar) is incremented, skip_bitmap (uint8 [B,Hq,nT,nT]) filled."""
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _dev(q, k, v, o, lse, skip_bitmap, skipped_tiles)
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape or o.shape != q.shape:
        raise ValueError("shape mismatch")
    for t in (q, k, v, o):
        if t.dtype != torch.bfloat16:
            raise TypeError("attn_prefill_blockskip takes bfloat16 tensors")
    nT = (S + 63) // 64
    if skip_bitmap is not None and (skip_bitmap.dtype != torch.uint8
                                    or skip_bitmap.shape != (B, Hq, nT, nT)):
        raise ValueError("skip_bitmap must be uint8 [B,Hq,nT,nT]")
    if skipped_tiles is not None and (skipped_tiles.numel() != 1 or skipped_tiles.element_size() != 8):
        raise ValueError("skipped_tiles must be one 64-bit integer")
    st = load().attn_prefill_blockskip(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                       S, D, float(scale), float(lam), int(tile),
                                       _ptr(skip_bitmap), _ptr(skipped_tiles), _stream(stream))
    _check(st, "attn_prefill_blockskip")


def attn_decode_workspace_bytes(num_seqs: int, Hq: int, D: int, max_blocks_per_seq: int,
                                block_size: int = 16) -> int:
    return int(load().attn_decode_workspace_bytes(num_seqs, Hq, D, max_blocks_per_seq,
                                                  block_size))


KV_LAYOUTS = {"rowmajor": 0, "mfma": 1}


def _pool_shapes(NB, Hkv, bs, D, layout):
    if layout == "rowmajor":
        return (NB, Hkv, bs, D), (NB, Hkv, bs, D)
    return (NB, Hkv, D // 8, bs, 8), (NB, Hkv, D, bs)


def _decode_check(q, k_pool, v_pool, block_table, seq_lens, block_size, o, lse, workspace,
                  layout):
    N, Hq, D = q.shape
    NB, Hkv = k_pool.shape[0], k_pool.shape[1]
    _dev(q, k_pool, v_pool, block_table, seq_lens, o, lse, workspace)
    if layout not in KV_LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    ks, vs = _pool_shapes(NB, Hkv, block_size, D, layout)
    if tuple(k_pool.shape) != ks or tuple(v_pool.shape) != vs or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != N or seq_lens.shape != (N,):
        raise ValueError("block_table must be [N, max_blocks], seq_lens [N]")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (N, Hq)):
        raise ValueError("lse must be float32 [N,Hq]")
    return N, Hq, Hkv, D, NB, workspace.numel() * workspace.element_size()


def attn_decode_paged(q, k_pool, v_pool, block_table, seq_lens, block_size: int, o, lse,
                      scale: float, workspace, stream=None, layout: str = "rowmajor") -> None:
    """Paged decode into caller-allocated o [N,Hq,D] and lse [N,Hq] (or None).
    ``layout`` names the pool layout: "rowmajor" or "mfma" (see include/attn.h)."""
    N, Hq, Hkv, D, NB, nbytes = _decode_check(q, k_pool, v_pool, block_table, seq_lens,
                                              block_size, o, lse, workspace, layout)
    st = load().attn_decode_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                  _ptr(seq_lens), int(block_size), KV_LAYOUTS[layout], _ptr(o),
                                  _ptr(lse), N, Hq, Hkv,
                                  D, NB, int(block_table.shape[1]), float(scale), _ptr(workspace),
                                  nbytes, _stream(stream))
    _check(st, "attn_decode_paged")


def attn_decode_paged_noalloc(q, k_pool, v_pool, block_table, seq_lens, block_size: int, o, lse,
                              scale: float, stream=None, layout: str = "rowmajor") -> None:
    """Paged decode into caller-allocated o and lse (or None) with the
    library's static scratch in place of a workspace (no device allocation
    in the call; requests larger than DECODE_STATIC_SCRATCH_BYTES raise)."""
    N, Hq, D = q.shape
    NB, Hkv = k_pool.shape[0], k_pool.shape[1]
    _dev(q, k_pool, v_pool, block_table, seq_lens, o, lse)
    if layout not in KV_LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    ks, vs = _pool_shapes(NB, Hkv, block_size, D, layout)
    if tuple(k_pool.shape) != ks or tuple(v_pool.shape) != vs or o.shape != q.shape:
        raise ValueError("shape mismatch")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != N or seq_lens.shape != (N,):
        raise ValueError("block_table must be [N, max_blocks], seq_lens [N]")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (N, Hq)):
        raise ValueError("lse must be float32 [N,Hq]")
    st = load().attn_decode_paged_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), int(block_size),
        KV_LAYOUTS[layout], _ptr(o), _ptr(lse), N, Hq, Hkv, D, NB, int(block_table.shape[1]),
        float(scale), _stream(stream))
    _check(st, "attn_decode_paged_noalloc")


def attn_decode_paged_blockskip(q, k_pool, v_pool, block_table, seq_lens, block_size: int, o,
                                lse, scale: float, lam: float, workspace, skip_bitmap=None,
                                skipped_blocks=None, stream=None, layout: str = "mfma") -> None:
    """Paged decode with block skipping (either pool layout); skip_bitmap is
    uint8 [N, Hkv, max_blocks] or None, skipped_blocks one 64-bit device
    integer (incremented) or None."""
    N, Hq, Hkv, D, NB, nbytes = _decode_check(q, k_pool, v_pool, block_table, seq_lens,
                                              block_size, o, lse, workspace, layout)
    MB = int(block_table.shape[1])
    _dev(skip_bitmap, skipped_blocks)
    if skip_bitmap is not None and (skip_bitmap.dtype != torch.uint8
                                    or skip_bitmap.shape != (N, Hkv, MB)):
        raise ValueError("skip_bitmap must be uint8 [N, Hkv, max_blocks]")
    if skipped_blocks is not None and (skipped_blocks.numel() != 1
                                       or skipped_blocks.element_size() != 8):
        raise ValueError("skipped_blocks must be one 64-bit integer")
    st = load().attn_decode_paged_blockskip(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), int(block_size),
        KV_LAYOUTS[layout], _ptr(o), _ptr(lse), N, Hq, Hkv, D, NB, MB, float(scale), float(lam),
        _ptr(skip_bitmap), _ptr(skipped_blocks), _ptr(workspace), nbytes, _stream(stream))
    _check(st, "attn_decode_paged_blockskip")


def attn_decode_paged_fp8(q, k_pool, v_pool, block_table, seq_lens, block_size: int, o, lse,
                          scale: float, k_scale: float, v_scale: float, workspace,
                          stream=None) -> None:
    """Paged decode over FP8 (E4M3) pools: uint8 k_pool / v_pool
    [NB, Hkv, 16 * D] in the byte order of include/attn.h, one scale each."""
    N, Hq, D = q.shape
    NB, Hkv = k_pool.shape[0], k_pool.shape[1]
    _dev(q, k_pool, v_pool, block_table, seq_lens, o, lse, workspace)
    if k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8:
        raise TypeError("FP8 pools are uint8 code tensors")
    if tuple(k_pool.shape) != (NB, Hkv, block_size * D) or v_pool.shape != k_pool.shape:
        raise ValueError("FP8 pools must be [NB, Hkv, block_size * D]")
    if o.shape != q.shape:
        raise ValueError("shape mismatch")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != N or seq_lens.shape != (N,):
        raise ValueError("block_table must be [N, max_blocks], seq_lens [N]")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (N, Hq)):
        raise ValueError("lse must be float32 [N,Hq]")
    st = load().attn_decode_paged_fp8(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), int(block_size),
        _ptr(o), _ptr(lse), N, Hq, Hkv, D, NB, int(block_table.shape[1]), float(scale),
        float(k_scale), float(v_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(st, "attn_decode_paged_fp8")


def attn_prefill_paged(q, cu_seqlens_q, k_pool, v_pool, block_table, seq_lens_k, o, lse,
                       max_seqlen_q: int, scale: float, block_size: int = 16, stream=None,
                       layout: str = "rowmajor") -> None:
    """Chunked / variable-length causal prefill over the paged cache into
    caller-allocated o [total_q, Hq, D] and lse [total_q, Hq] (or None)."""
    total_q, Hq, D = q.shape
    N = int(seq_lens_k.shape[0])
    NB, Hkv = k_pool.shape[0], k_pool.shape[1]
    _dev(q, cu_seqlens_q, k_pool, v_pool, block_table, seq_lens_k, o, lse)
    if layout not in KV_LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    ks, vs = _pool_shapes(NB, Hkv, block_size, D, layout)
    if tuple(k_pool.shape) != ks or tuple(v_pool.shape) != vs or o.shape != q.shape:
        raise ValueError("shape mismatch")
    for t in (cu_seqlens_q, block_table, seq_lens_k):
        if t.dtype != torch.int32:
            raise TypeError("cu_seqlens_q, block_table and seq_lens_k must be int32")
    if cu_seqlens_q.shape != (N + 1,) or block_table.dim() != 2 or block_table.shape[0] != N:
        raise ValueError("cu_seqlens_q must be [N+1], block_table [N, max_blocks]")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (total_q, Hq)):
        raise ValueError("lse must be float32 [total_q, Hq]")
    st = load().attn_prefill_paged(
        _ptr(q), _ptr(cu_seqlens_q), total_q, int(max_seqlen_q), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), _ptr(seq_lens_k), int(block_size), KV_LAYOUTS[layout], _ptr(o),
        _ptr(lse), N, Hq, Hkv, D, NB, int(block_table.shape[1]), float(scale), _stream(stream))
    _check(st, "attn_prefill_paged")


# ------------------------------------------------------ allocating wrappers

def prefill(q, k, v, causal: bool = True, scale: Optional[float] = None,
            with_lse: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Allocate O (and LSE) and run the bf16 or fp32 prefill chosen by q.dtype."""
    B, Hq, S, D = q.shape
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if with_lse else None
    if q.dtype == torch.float32:
        attn_prefill_f32(q, k, v, o, lse, causal, scale)
    else:
        attn_prefill(q, k, v, o, lse, causal, scale)
    return o, lse


def prefill_blockskip(q, k, v, scale: Optional[float] = None, lam: float = 1e-3,
                      with_bitmap: bool = True):
    """Returns (O, LSE, skip bitmap or None, skipped-tile count tensor)."""
    B, Hq, S, D = q.shape
    if scale is None:
        scale = D ** -0.5
    nT = (S + 63) // 64
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    bm = torch.zeros((B, Hq, nT, nT), dtype=torch.uint8, device=q.device) if with_bitmap else None
    cnt = torch.zeros(1, dtype=torch.int64, device=q.device)
    attn_prefill_blockskip(q, k, v, o, lse, scale, lam, 64, bm, cnt)
    return o, lse, bm, cnt


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, block_size: int = 16,
                 scale: Optional[float] = None, workspace=None, layout: str = "rowmajor"):
    """Allocate O, LSE (and the workspace unless given) and run the paged decode."""
    N, Hq, D = q.shape
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = attn_decode_workspace_bytes(N, Hq, D, int(block_table.shape[1]), block_size)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    attn_decode_paged(q, k_pool, v_pool, block_table, seq_lens, block_size, o, lse, scale,
                      workspace, layout=layout)
    return o, lse


def decode_paged_noalloc(q, k_pool, v_pool, block_table, seq_lens, block_size: int = 16,
                         scale: Optional[float] = None, layout: str = "rowmajor"):
    """Allocate O and LSE and run the paged decode on the library's static
    scratch (the call itself allocates no workspace)."""
    N, Hq, D = q.shape
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    attn_decode_paged_noalloc(q, k_pool, v_pool, block_table, seq_lens, block_size, o, lse, scale,
                              layout=layout)
    return o, lse


def decode_paged_blockskip(q, k_pool, v_pool, block_table, seq_lens, lam: float,
                           block_size: int = 16, scale: Optional[float] = None, workspace=None,
                           layout: str = "mfma"):
    """Allocate O, LSE, the skip bitmap and counter (and the workspace unless
    given) and run the block-skip paged decode on pools in ``layout``.
    Returns (o, lse, skip_bitmap, skipped_blocks)."""
    N, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    bm = torch.zeros((N, Hkv, int(block_table.shape[1])), dtype=torch.uint8, device=q.device)
    cnt = torch.zeros(1, dtype=torch.int64, device=q.device)
    if workspace is None:
        nbytes = attn_decode_workspace_bytes(N, Hq, D, int(block_table.shape[1]), block_size)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    attn_decode_paged_blockskip(q, k_pool, v_pool, block_table, seq_lens, block_size, o, lse,
                                scale, lam, workspace, bm, cnt, layout=layout)
    return o, lse, bm, cnt


def decode_paged_fp8(q, k_pool, v_pool, block_table, seq_lens, k_scale: float, v_scale: float,
                     block_size: int = 16, scale: Optional[float] = None, workspace=None):
    """Allocate O, LSE (and the workspace unless given) and run the paged
    decode over FP8 pools."""
    N, Hq, D = q.shape
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = attn_decode_workspace_bytes(N, Hq, D, int(block_table.shape[1]), block_size)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    attn_decode_paged_fp8(q, k_pool, v_pool, block_table, seq_lens, block_size, o, lse, scale,
                          k_scale, v_scale, workspace)
    return o, lse


def prefill_paged(q, cu_seqlens_q, k_pool, v_pool, block_table, seq_lens_k, max_seqlen_q: int,
                  scale: Optional[float] = None, block_size: int = 16):
    """Allocate O and LSE and run the chunked prefill over a row-major paged
    cache.  Returns (o [total_q, Hq, D], lse [total_q, Hq])."""
    total_q, Hq, D = q.shape
    if scale is None:
        scale = D ** -0.5
    o = torch.empty_like(q)
    lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    attn_prefill_paged(q, cu_seqlens_q, k_pool, v_pool, block_table, seq_lens_k, o, lse,
                       max_seqlen_q, scale, block_size)
    return o, lse
