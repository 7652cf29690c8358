"""C-ABI checks that need no GPU: the library loads, exports every function
include/attn.h declares, and rejects invalid arguments before touching HIP."""
import ctypes
import os
import re

import pytest

import attention_flash_attn_fwd_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(A.lib_path()),
                                reason="libattn.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*(attn_[a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


def test_header_lists_the_entry_points():
    names = _declared()
    for need in ("attn_prefill", "attn_prefill_f32", "attn_prefill_blockskip",
                 "attn_decode_paged", "attn_decode_paged_blockskip", "attn_prefill_paged",
                 "attn_decode_paged_fp8", "attn_decode_paged_noalloc",
                 "attn_decode_workspace_bytes", "attn_status_string", "attn_arch_supported"):
        assert need in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(A.lib_path())
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings_and_arch_names():
    assert A.attn_status_string(0) == "ok"
    for st in (-1, -2, -3, -4, -5, -6, -7):
        assert A.attn_status_string(st) not in ("ok", "unknown status")
    assert A.attn_status_string(7) == "unknown status"
    assert A.attn_arch_supported("gfx950")
    assert A.attn_arch_supported("gfx950:sramecc+:xnack-")
    for bad in ("gfx942", "gfx9500", "gfx95", "", "gfx90a:xnack+"):
        assert not A.attn_arch_supported(bad)
    assert A.load().attn_arch_supported(None) == 0


def _pre(lib, name="attn_prefill", **kw):
    a = dict(q=8, k=8, v=8, o=8, lse=None, B=1, Hq=4, Hkv=2, S=16, D=64, causal=1, scale=0.125)
    a.update(kw)
    return getattr(lib, name)(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                              a["S"], a["D"], a["causal"], a["scale"], None)


@pytest.mark.parametrize("name", ["attn_prefill", "attn_prefill_f32"])
def test_prefill_validation_without_device(name):
    lib = A.load()
    assert _pre(lib, name, q=None) == -1
    assert _pre(lib, name, o=None) == -1
    assert _pre(lib, name, B=0) == -1
    assert _pre(lib, name, S=0) == -1
    assert _pre(lib, name, Hq=3, Hkv=2) == -1
    assert _pre(lib, name, causal=2) == -1
    assert _pre(lib, name, scale=0.0) == -1
    assert _pre(lib, name, scale=float("nan")) == -1
    assert _pre(lib, name, scale=-1.0) == -1
    assert _pre(lib, name, D=96) == -2
    assert _pre(lib, name, D=256) == -2


def test_blockskip_validation_without_device():
    lib = A.load()

    def call(lam=1e-3, tile=64, q=8, Hq=4):
        return lib.attn_prefill_blockskip(q, 8, 8, 8, None, 1, Hq, 2, 128, 128, 0.1, lam, tile,
                                          None, None, None)
    assert call(lam=0.0) == -1
    assert call(lam=1.0) == -1
    assert call(lam=-0.5) == -1
    assert call(tile=128) == -2
    assert call(q=None) == -1
    assert call(Hq=3) == -1


def test_decode_workspace_and_validation_without_device():
    lib = A.load()
    # 64 sequences, 32 query heads, D=128, 256 blocks of 16 tokens -> 8 splits of 512 tokens
    assert A.attn_decode_workspace_bytes(64, 32, 128, 256, 16) == 64 * 32 * 8 * 129 * 4
    assert A.attn_decode_workspace_bytes(1, 1, 64, 33, 16) == 1 * 1 * 2 * 65 * 4
    assert A.attn_decode_workspace_bytes(0, 32, 128, 256, 16) == 0
    need = A.attn_decode_workspace_bytes(2, 8, 128, 4, 16)

    def call(**kw):
        a = dict(q=8, kp=8, vp=8, bt=8, sl=8, bs=16, lay=1, o=8, N=2, Hq=8, Hkv=2, D=128, NB=8,
                 MB=4, scale=0.1, ws=256, wsb=need)
        a.update(kw)
        return lib.attn_decode_paged(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["bs"], a["lay"],
                                     a["o"],
                                     None, a["N"], a["Hq"], a["Hkv"], a["D"], a["NB"], a["MB"],
                                     a["scale"], a["ws"], a["wsb"], None)
    assert call(bt=None) == -1
    assert call(sl=None) == -1
    assert call(N=0) == -1
    assert call(Hq=6, Hkv=4) == -1
    assert call(NB=0) == -1
    assert call(scale=float("inf")) == -1
    assert call(lay=2) == -1
    assert call(lay=-1) == -1
    assert call(bs=32) == -2
    assert call(D=80) == -2
    assert call(Hq=64, Hkv=2) == -2          # group of 32 query heads
    assert call(ws=None) == -4
    assert call(wsb=need - 1) == -4
    assert call(ws=260) == -4                # misaligned workspace


def test_decode_noalloc_validation_without_device():
    """The allocation-free decode validates like attn_decode_paged and rejects
    a request whose split-KV scratch exceeds the static array, before any HIP
    call."""
    lib = A.load()
    hdr = open(HEADER).read()
    assert re.search(r"#define ATTN_DECODE_STATIC_SCRATCH_BYTES \(16u << 20\)", hdr)
    assert A.DECODE_STATIC_SCRATCH_BYTES == 16 << 20

    def call(**kw):
        a = dict(q=8, kp=8, vp=8, bt=8, sl=8, bs=16, lay=1, o=8, N=2, Hq=8, Hkv=2, D=128, NB=8,
                 MB=4, scale=0.1)
        a.update(kw)
        return lib.attn_decode_paged_noalloc(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["bs"],
                                             a["lay"], a["o"], None, a["N"], a["Hq"], a["Hkv"],
                                             a["D"], a["NB"], a["MB"], a["scale"], None)
    assert call(bt=None) == -1
    assert call(N=0) == -1
    assert call(Hq=6, Hkv=4) == -1
    assert call(lay=2) == -1
    assert call(bs=32) == -2
    assert call(D=80) == -2
    # 64 sequences x 32 heads x D=128: rows of up to 480 blocks (15 splits of
    # 512 tokens, 64*32*15*129*4 B) fit in 16 MiB, 481 blocks and more do not
    lim = A.DECODE_STATIC_SCRATCH_BYTES
    assert A.attn_decode_workspace_bytes(64, 32, 128, 480, 16) <= lim
    assert A.attn_decode_workspace_bytes(64, 32, 128, 481, 16) > lim
    for mb in (256, 480, 481, 512, 1024):
        need = A.attn_decode_workspace_bytes(64, 32, 128, mb, 16)
        st = call(N=64, Hq=32, Hkv=8, MB=mb)
        if need > lim:
            assert st == -7, (mb, need)
        else:
            assert st not in (-7, -4, -1, -2), (mb, need, st)
    assert "static decode scratch" in A.attn_status_string(-7)


def test_decode_blockskip_validation_without_device():
    lib = A.load()
    need = A.attn_decode_workspace_bytes(2, 8, 128, 4, 16)

    def call(**kw):
        a = dict(q=8, kp=8, vp=8, bt=8, sl=8, bs=16, lay=1, o=8, N=2, Hq=8, Hkv=2, D=128, NB=8,
                 MB=4, scale=0.1, lam=1e-3, ws=256, wsb=need)
        a.update(kw)
        return lib.attn_decode_paged_blockskip(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["bs"],
                                               a["lay"], a["o"], None, a["N"], a["Hq"], a["Hkv"],
                                               a["D"], a["NB"], a["MB"], a["scale"], a["lam"],
                                               None, None, a["ws"], a["wsb"], None)
    assert call(lam=0.0) == -1
    assert call(lam=1.0) == -1
    assert call(lam=float("nan")) == -1
    assert call(lay=0) not in (-1, -2)  # row-major pools are supported too
    assert call(lay=3) == -1
    assert call(bt=None) == -1
    assert call(D=96) == -2
    assert call(ws=None) == -4


def test_prefill_paged_validation_without_device():
    lib = A.load()

    def call(**kw):
        a = dict(q=8, cu=8, tq=40, mq=20, kp=8, vp=8, bt=8, sk=8, bs=16, lay=0, o=8, N=2, Hq=8,
                 Hkv=2, D=128, NB=8, MB=4, scale=0.1)
        a.update(kw)
        return lib.attn_prefill_paged(a["q"], a["cu"], a["tq"], a["mq"], a["kp"], a["vp"], a["bt"],
                                      a["sk"], a["bs"], a["lay"], a["o"], None, a["N"], a["Hq"],
                                      a["Hkv"], a["D"], a["NB"], a["MB"], a["scale"], None)
    assert call(cu=None) == -1
    assert call(tq=0) == -1
    assert call(mq=0) == -1
    assert call(Hq=6, Hkv=4) == -1
    assert call(scale=-1.0) == -1
    assert call(lay=5) == -1
    assert call(lay=1) == -2           # MFMA-native pools: not supported here
    assert call(bs=32) == -2
    assert call(D=96) == -2
    assert call(Hq=70000, Hkv=70000) == -2   # pool block bytes must stay 32-bit


def test_decode_fp8_validation_without_device():
    lib = A.load()
    need = A.attn_decode_workspace_bytes(2, 8, 128, 4, 16)

    def call(**kw):
        a = dict(q=8, kp=8, vp=8, bt=8, sl=8, bs=16, o=8, N=2, Hq=8, Hkv=2, D=128, NB=8, MB=4,
                 scale=0.1, ks=0.01, vs=0.02, ws=256, wsb=need)
        a.update(kw)
        return lib.attn_decode_paged_fp8(a["q"], a["kp"], a["vp"], a["bt"], a["sl"], a["bs"],
                                         a["o"], None, a["N"], a["Hq"], a["Hkv"], a["D"], a["NB"],
                                         a["MB"], a["scale"], a["ks"], a["vs"], a["ws"], a["wsb"],
                                         None)
    assert call(ks=0.0) == -1
    assert call(vs=-1.0) == -1
    assert call(ks=float("nan")) == -1
    assert call(vs=float("inf")) == -1
    assert call(kp=None) == -1
    assert call(Hq=6, Hkv=4) == -1
    assert call(bs=32) == -2
    assert call(D=96) == -2
    assert call(Hq=64, Hkv=2) == -2
    assert call(ws=None) == -4
    assert call(wsb=need - 1) == -4


def test_binding_device_check(monkeypatch):
    """The binding takes tensors of one GPU, the current one (stand-ins here:
    only the device attribute is read, and the current device is patched)."""
    import types
    import torch

    def t(dev):
        return types.SimpleNamespace(device=torch.device(dev))

    monkeypatch.setattr(torch.cuda, "current_device", lambda: 1)
    A._dev(t("cuda:1"), None, t("cuda:1"))          # same GPU as the current one
    with pytest.raises(ValueError, match="current device"):
        A._dev(t("cuda:0"), t("cuda:0"))
    with pytest.raises(ValueError, match="one GPU"):
        A._dev(t("cuda:1"), t("cuda:0"))
    with pytest.raises(ValueError, match="on the GPU"):
        A._dev(t("cuda:1"), t("cpu"))
    A._dev(None, None)                              # nothing to check
