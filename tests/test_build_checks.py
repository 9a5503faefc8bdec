"""Checks on the compiled gfx950 code that need no GPU.

The small-batch W4A16 kernel waits for its staged activations with a hand-counted
s_waitcnt vmcnt(N): N must not exceed the number of vector-memory instructions the
compiler actually issued after the staging loads (it may merge adjacent loads), or the
wait would let the kernel read the staging area early."""
import os
import re
import subprocess

import pytest

from bit_floating_point_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")
def test_small_kernel_waits_are_lower_bounds(tmp_path):
    asm = tmp_path / "w16.s"
    cmd = [B.HIPCC] + B.CFLAGS + ["--cuda-device-only", "-S", os.path.join(B.CSRC, "gemm_w4a16.hip"), "-o", str(asm)]
    subprocess.run(cmd, check=True, capture_output=True)
    s = asm.read_text()
    names = re.findall(r"^(_ZN3fp418w4a16_small_kernel\w+):", s, re.M)
    assert len(names) > 40
    for name in names:
        body = s[s.index(name + ":"):s.index(".Lfunc_end", s.index(name + ":"))]
        loads, first = 0, None
        for line in body.split("\n"):
            t = line.strip()
            if t.startswith("buffer_load") and " lds" not in t:
                loads += 1
            m = re.match(r"s_waitcnt vmcnt\((\d+)\)", t)
            if m:
                first = int(m.group(1))
                break
        assert first is not None and first <= loads, (name, loads, first)
