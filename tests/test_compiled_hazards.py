"""Checks on the gfx950 machine code of the HIP kernels (CPU only: hipcc
cross-compiles to assembly here).

gfx950 does not interlock a VALU read of the result of a VGPR-form MFMA: the
instruction stream must leave enough wait states (s_nop) between them.  The
compiler counts them within a basic block, but a read placed right after a
branch that skips a few instructions (for example a conditional tail mask)
was found to get none on the taken path, so the read saw stale register
contents.  This test compiles every kernel source with the library's own
flags and follows both branch directions from each MFMA for a few
instructions, failing if its destination registers are read by a VALU
instruction before `NEED` wait states have passed (8-pass MFMAs need more
than that; the bound is deliberately loose, so only clear misses fail).
"""
import os
import re
import subprocess

import pytest

from attention_flash_attn_fwd_amd import _build

NEED = 8
KERNELS = ["prefill_bf16.hip", "decode_paged.hip"]


def _hipcc():
    try:
        return _build._hipcc()
    except RuntimeError:
        return None


def _regs(tok):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]|(?<![a-z_])v(\d+)", tok):
        if m.group(3):
            out.add(int(m.group(3)))
        else:
            out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _misses(asm):
    """(function, mfma line, reading line, wait states) for every VALU read
    of an MFMA destination reached with fewer than NEED wait states."""
    found = []
    for fm in re.finditer(r"^(_Z\S+):[^\n]*\n(.*?)\.Lfunc_end", asm, flags=re.S | re.M):
        name, body = fm.group(1), fm.group(2).split("\n")
        labels = {l.split(":")[0]: i for i, l in enumerate(body) if re.match(r"^\.LBB\S+:", l)}
        for i, line in enumerate(body):
            m = re.match(r"\s*v_mfma\S*\s+(v\[\d+:\d+\]|v\d+),", line)
            if not m:
                continue
            dst = _regs(m.group(1))
            stack, seen = [(i + 1, 0, 0)], set()
            while stack:
                j, ws, steps = stack.pop()
                if (j, ws) in seen or steps > 12 or j >= len(body):
                    continue
                seen.add((j, ws))
                t = body[j].strip()
                if not t or t[0] in ";.%":
                    stack.append((j + 1, ws, steps))
                    continue
                op = t.split()[0]
                if op == "s_nop":
                    stack.append((j + 1, ws + int(t.split()[1]) + 1, steps + 1))
                    continue
                if op.startswith("v_") and not op.startswith("v_mfma") and " " in t:
                    srcs = _regs(",".join(t.split(None, 1)[1].split(",")[1:]))
                    if srcs & dst and ws < NEED:
                        found.append((name, i, j, ws))
                        continue
                if op.startswith("s_cbranch") or op == "s_branch":
                    tgt = t.split()[1]
                    if tgt in labels:
                        stack.append((labels[tgt] + 1, ws + 1, steps + 1))
                    if op == "s_branch":
                        continue
                if op == "s_endpgm":
                    continue
                stack.append((j + 1, ws + 1, steps + 1))
    return found


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
@pytest.mark.parametrize("src", KERNELS)
def test_no_mfma_result_read_without_wait_states(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [_hipcc(), *_build._flags(src), "--cuda-device-only", "-S",
           os.path.join(_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    misses = _misses(out.read_text())
    assert not misses, f"MFMA results read too early in {src}: {misses[:5]}"


def test_scanner_flags_a_read_after_a_branch():
    """The scanner itself: a read of an MFMA result right after a taken
    branch with no s_nop is flagged; the same read behind s_nop 7 + s_nop 1
    (10 wait states) is not."""
    bad = """_Zk:
\tv_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[12:15], 0
\ts_cbranch_scc1 .LBB0_2
\tv_mov_b32_e32 v1, 0
.LBB0_2:
\tv_max_f32_e32 v3, v7, v7
\ts_endpgm
.Lfunc_end0:
"""
    good = bad.replace("\ts_cbranch_scc1", "\ts_nop 7\n\ts_nop 1\n\ts_cbranch_scc1")
    assert _misses(bad)
    assert not _misses(good)
