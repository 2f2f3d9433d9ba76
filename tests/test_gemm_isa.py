"""The GEMM ring kernel reads its MFMA fragments from LDS with explicit
ds_read instructions (the compiler does not see the direct-to-LDS copies, so
the waits are the kernel's own).  Its correctness rests on one property of
the generated code: no instruction reads a fragment register between the
ds_read that fills it and the following `s_waitcnt lgkmcnt(0)`.  This test
compiles the kernel for gfx950 (host only, no GPU) and checks that property
in every instantiation.
"""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    path = os.path.join(ROOT, "deterministic_paged_attention_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_bi_build_isa", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _kernels(asm: str):
    for m in re.finditer(r"^(_Z\S*gemm_(?:ring|skinny)_kernel\S*?):[^\n]*\n(.*?)^\.Lfunc_end", asm, re.S | re.M):
        yield m.group(1), m.group(2)


def _regs(text):
    for mm in re.finditer(r"v\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if mm.group(1):
            yield from range(int(mm.group(1)), int(mm.group(2)) + 1)
        else:
            yield int(mm.group(3))


def early_reads(body: str):
    """Instructions that read a register whose ds_read has not been waited for."""
    pending, bad = set(), []
    for line in body.split("\n"):
        t = line.strip()
        if not t or t.startswith((";", ".")):
            continue
        m = re.match(r"ds_read\w*\s+(v\[\d+:\d+\]|v\d+)\s*,", t)
        if m:
            pending |= set(_regs(m.group(1)))
            continue
        if t.startswith("s_waitcnt") and "lgkmcnt(0)" in t:
            pending.clear()
            continue
        if pending and " " in t:
            operands = t.split(None, 1)[1].split(",")
            if set(_regs(",".join(operands[1:]))) & pending:
                bad.append(t)
    return bad


def test_early_read_detector_flags_a_planted_use():
    body = "ds_read_b128 v[4:7], v1\nv_mov_b32 v9, v5\ns_waitcnt lgkmcnt(0)\nv_mov_b32 v10, v6\n"
    assert early_reads(body) == ["v_mov_b32 v9, v5"]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_gemm_fragments_are_waited_for_before_use(tmp_path):
    b = _build_module()
    out = tmp_path / "gemm.s"
    cmd = [b.HIPCC, *[f for f in b.FLAGS if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(b.CSRC, "gemm.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = list(_kernels(out.read_text()))
    assert len(kernels) >= 4
    for name, body in kernels:
        assert "ds_read" in body, name
        assert early_reads(body) == [], name
